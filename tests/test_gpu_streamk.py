"""GPU parity of the stream-K mode (PGEMM_SCHED_STREAMK) through the C ABI.

Stream-K is the tail handling that creates work instead of idling CUs: with
T = W*G + R tiles, W whole waves run as in the static mode and the k-steps
of the R tail tiles are split over the workgroups, with a fix-up launch
adding the split tiles' fp32 partials in k order (the KernelWiki page
"Persistent Kernels with Cluster Launch Control", "Choosing between static
and CLC scheduling", notes that neither of its schedulers creates work at
the tail). The cases cover every shape of split the planner makes:

* W = 0 (fewer tiles than workgroups: every tile split), W >= 1 (whole
  waves plus a split tail), 256 x 256 and 128 x 128 tiles;
* pieces that straddle tile boundaries (k-step pairs per tile not a
  multiple of the piece length), and tiles too short to split (no fix-up);
* ragged M and N edges inside split tiles, and a K tail;
* fp16, bf16 and fp8 (e4m3) inputs.

Per case: small-integer inputs bit-exact against the oracle (every partial
sum is an integer below 2^24, exact in fp32 however the k-range is split);
uniform[-1,1] inputs within the oracle bound; every tile visited exactly
once; owner log: whole tiles of the first waves at t mod G, split tiles
marked as stored by the fix-up (-1 - s); a rerun bitwise identical (the
fix-up adds the partials in a fixed order).
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

SK = 4
DT = {"f16": 0, "bf16": 1, "e4m3fn": 2}
OUT = {"f16": ("f16", torch.float16), "bf16": ("bf16", torch.bfloat16), "e4m3fn": ("bf16", torch.bfloat16)}
TOL = {"f16": 2e-3, "bf16": 2e-3, "e4m3fn": 1e-2}
TILES = {256: 1, 128: 2}  # PGEMM_TILE_256, PGEMM_TILE_128

# (dtype, M, N, K, tile, grid_multiple, what it exercises)
CASES = [
    ("f16", 512, 512, 2048, 256, 0, "W=0: 4 tiles of 256^2, each split over 4 workgroups"),
    ("bf16", 1000, 1032, 4000, 128, 0, "W=0, ragged edges in split tiles, K tail"),
    ("e4m3fn", 768, 1024, 8192, 128, 0, "W=0, fp8 steps of 128"),
    ("f16", 640, 640, 576, 128, 0, "5 pairs per tile, pieces of ~4: straddle tile boundaries"),
    ("f16", 1024, 1024, 64, 128, 0, "1 pair per tile: nothing split, no fix-up"),
    ("f16", 4096, 4096, 512, 256, 0, "T = 256 = G: no tail, one static launch, no fix-up"),
    ("f16", 2176, 2176, 1024, 128, 1, "W=1 whole wave of 256 + 33 tail tiles split in two"),
    ("bf16", 3000, 2056, 2000, 128, 1, "W=1, R=152 tail tiles, ragged edges, K tail"),
    ("f16", 4352, 4352, 1024, 256, 0, "256^2 tiles, W=1, R=33 tail tiles split in two"),
    ("e4m3fn", 2304, 2176, 2048, 128, 1, "fp8, W=1, R=50 tail tiles split in two"),
]


@pytest.fixture(scope="module")
def pg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_macro_amd as pg
    return pg


@pytest.fixture(scope="module")
def handles(pg):
    """One handle per (tile, mainloop): the automatic wave schedule (ping-pong for the whole
    waves of long k-loops) and lockstep waves forced."""
    hs = {}
    for tile, code in TILES.items():
        for ml in (0, 1):
            h = pg.pgemm_create(0)
            pg.pgemm_set_tile_config(h, code)
            pg.pgemm_set_mainloop(h, ml)
            hs[(tile, ml)] = h
    yield hs
    for h in hs.values():
        pg.pgemm_destroy(h)


def say(msg):
    print(msg, flush=True)


def run_sk(pg, h, Ad, Bd, M, N, K, dtype, gm, log=True):
    dev = Ad.device
    info = pg.pgemm_query_launch(h, M, N, K, DT[dtype], SK, gm)
    C = torch.full((M, N), float("nan"), dtype=OUT[dtype][1], device=dev)
    visits = owner = None
    if log:
        visits = torch.zeros(info["tiles"], dtype=torch.int32, device=dev)
        owner = torch.full((info["tiles"],), -1, dtype=torch.int32, device=dev)
        pg.pgemm_set_tile_counter(h, visits)
        pg.pgemm_set_owner_log(h, owner)
    try:
        pg.pgemm_run(h, Ad, Bd, C, M, N, K, DT[dtype], SK, gm)
        torch.cuda.synchronize()
    finally:
        if log:
            pg.pgemm_set_tile_counter(h, None)
            pg.pgemm_set_owner_log(h, None)
    return C, info, (visits.cpu().numpy() if log else None), (owner.cpu().numpy() if log else None)


@pytest.mark.parametrize("mainloop", [0, 1], ids=["auto", "lockstep"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-t{c[4]}-g{c[5]}" for c in CASES])
def test_streamk_parity(pg, handles, case, mainloop):
    dtype, M, N, K, tile, gm, what = case
    h = handles[(tile, mainloop)]
    dev = torch.device("cuda:0")
    split = pg.pgemm_query_streamk(h, M, N, K, DT[dtype], gm)
    info = pg.pgemm_query_launch(h, M, N, K, DT[dtype], SK, gm)
    say(f"case stream-K {dtype} {M}x{N}x{K} tile {tile} gm {gm}: {what}; {split} grid {info['grid']}")
    T, G = info["tiles"], info["grid"]
    assert info["fast_path"] == 1 and info["bm"] == tile
    R = split["split_tiles"]
    assert split["whole_tiles"] + R == T
    if R:
        kp = ((K + info["bk"] - 1) // info["bk"] + 1) // 2
        assert 1 <= split["split_groups"] <= min(R * kp, max(G, split["split_groups"]))
        if split["pieces_split"]:
            assert split["workspace_bytes"] == (split["split_groups"] + R) * info["bm"] * info["bn"] * 4
    if "no fix-up" in what:
        assert split["pieces_split"] == 0 and split["workspace_bytes"] == 0
    elif "split" in what or "straddle" in what:
        assert split["pieces_split"] > 0

    # small integers: bit-exact, every tile once, owner log, rerun identical
    A, B = si.operands(M, N, K, dtype, "small_int", workload=21)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), dtype), OUT[dtype][0])
    Ad, Bd = A.to(dev), B.to(dev)
    C, _, visits, owner = run_sk(pg, h, Ad, Bd, M, N, K, dtype, gm)
    got = si.bits(C.cpu())
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    assert np.array_equal(visits, np.ones(T, np.int32)), np.nonzero(visits != 1)[0][:10]
    whole = T - R
    W = whole // G if G else 0
    if W:
        assert np.array_equal(owner[:whole], np.arange(whole) % G)
    tail = owner[whole:]
    by_fixup = np.nonzero(tail < 0)[0]
    assert len(by_fixup) == split["pieces_split"]
    assert np.array_equal(tail[by_fixup], -1 - by_fixup)  # split tiles: stored by the fix-up
    assert np.all(tail[tail >= 0] < max(split["split_groups"], 1))  # whole tail tiles: tail-launch workgroups

    # nothing cut into pieces: the same tile bodies as the static mode, so the same bits
    if split["pieces_split"] == 0:
        Cs = torch.full((M, N), float("nan"), dtype=OUT[dtype][1], device=dev)
        pg.pgemm_run(h, Ad, Bd, Cs, M, N, K, DT[dtype], 1, gm)
        torch.cuda.synchronize()
        assert torch.equal(Cs.view(torch.int16), C.view(torch.int16))

    # uniform inputs: within the bound, and a rerun gives the same bits
    A, B = si.operands(M, N, K, dtype, "uniform", workload=22)
    ref = oracle.gemm(si.bits(A), si.bits(B), dtype)
    Ad, Bd = A.to(dev), B.to(dev)
    C1, _, _, _ = run_sk(pg, h, Ad, Bd, M, N, K, dtype, gm, log=False)
    err = oracle.normwise_error(si.bits(C1.cpu()), OUT[dtype][0], ref)
    assert err <= TOL[dtype], err
    C2, _, _, _ = run_sk(pg, h, Ad, Bd, M, N, K, dtype, gm, log=False)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


def test_workspace_grows_and_is_reused(pg):
    """One handle: a run needing a small workspace, one needing a larger one
    (the handle reallocates), then the small one again (reused, no
    reallocation needed); every result bit-exact."""
    dev = torch.device("cuda:0")
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(h, pg.PGEMM_TILE_128)
        shapes = [(512, 512, 1024), (1024, 1536, 2048), (512, 512, 1024), (384, 640, 4096)]
        need = [pg.pgemm_query_streamk(h, M, N, K, 0, 0)["workspace_bytes"] for M, N, K in shapes]
        assert need[1] > need[0] > 0
        for i, (M, N, K) in enumerate(shapes):
            say(f"case workspace {i}: {M}x{N}x{K} needs {need[i]} bytes")
            A, B = si.operands(M, N, K, "f16", "small_int", workload=30 + i)
            want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
            C, _, visits, _ = run_sk(pg, h, A.to(dev), B.to(dev), M, N, K, "f16", 0)
            assert np.array_equal(si.bits(C.cpu()), want), i
            assert np.all(visits == 1)
    finally:
        pg.pgemm_destroy(h)


def test_generic_body_runs_streamk_as_static(pg):
    """Unaligned operands (N not a multiple of 8) take the 64 x 64 generic
    body, which has no split: the mode reports no tail tiles and is exact."""
    dev = torch.device("cuda:0")
    h = pg.pgemm_create(0)
    try:
        M, N, K = 300, 257, 700
        split = pg.pgemm_query_streamk(h, M, N, K, 0, 0)
        assert split["split_tiles"] == 0 and split["workspace_bytes"] == 0
        A, B = si.operands(M, N, K, "f16", "small_int", workload=40)
        want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
        C, info, visits, _ = run_sk(pg, h, A.to(dev), B.to(dev), M, N, K, "f16", 0)
        assert info["fast_path"] == 0
        assert np.array_equal(si.bits(C.cpu()), want)
        assert np.all(visits == 1)
    finally:
        pg.pgemm_destroy(h)


def test_streamk_with_xcd_remap_and_a_deep_split(pg):
    """Two corners of the split: (1) the XCD-aware tile remap on, where the
    whole-wave launch covers only the first W*G tiles (the remap's chunk, the
    CU count, divides W*G, so its tiles map exactly as in one launch); (2) a
    single tile whose K is cut into a hundred or more pieces, all added by one
    fix-up workgroup column. Small integers: bit-exact."""
    dev = torch.device("cuda:0")
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(h, pg.PGEMM_TILE_128)
        pg.pgemm_set_tile_order(h, 4, True)
        for (M, N, K, gm) in [(2176, 2176, 1024, 1), (128, 128, 65536, 0)]:
            split = pg.pgemm_query_streamk(h, M, N, K, 0, gm)
            say(f"case stream-K remap/deep {M}x{N}x{K} gm {gm}: {split}")
            assert split["pieces_split"] > 0
            A, B = si.operands(M, N, K, "f16", "small_int", workload=50)
            want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
            C, info, visits, _ = run_sk(pg, h, A.to(dev), B.to(dev), M, N, K, "f16", gm)
            assert np.array_equal(si.bits(C.cpu()), want)
            assert np.all(visits == 1)
        deep = pg.pgemm_query_streamk(h, 128, 128, 65536, 0, 0)
        assert deep["split_tiles"] == 1 and deep["split_groups"] >= 100
    finally:
        pg.pgemm_destroy(h)
