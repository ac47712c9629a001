"""GPU checks of the tile trace (pgemm_set_tile_trace), through the C ABI.

The trace runs a separate instantiation of the tile body, so the first
check is that it computes the same C bits as the untraced kernel. Then,
per scheduling mode and macro tile:
* every tile has an entry, and its workgroup id equals the owner log of the
  same run (stream-K split tiles: -1 - s, stored by the fix-up);
* start <= end, and the XCD id is one of the 8;
* workgroups are dealt round-robin over the XCDs (one rotation per launch);
* the tiles one workgroup ran follow each other without gaps or overlap:
  in start order, each tile starts at the clock value its predecessor
  ended at (the workgroup takes one reading per tile boundary);
* in the static mode a workgroup's tiles come in its fixed order t, t+G, ...
* a trace shorter than the run's tile count is rejected before launching.
"""
import warnings

import numpy as np
import pytest
import torch

import seeded_inputs as si

pytestmark = pytest.mark.gpu

# (tile config, mainloop): the 256 x 256 tile with lockstep waves and in ping-pong, the 256 x 128
# tile of the producer-wave body (stream-K keeps the lockstep 256 x 256 body), and 128 x 128
TILES = {"t256_lockstep": (1, 1), "t256_pingpong": (1, 2), "t256x128_producer": (1, 3), "t128": (2, 0)}


@pytest.fixture(scope="module")
def pg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_macro_amd as pg
    return pg


@pytest.fixture(scope="module", params=sorted(TILES))
def handle(pg, request):
    h = pg.pgemm_create(0)
    pg.pgemm_set_tile_config(h, TILES[request.param][0])
    pg.pgemm_set_mainloop(h, TILES[request.param][1])
    yield h
    pg.pgemm_destroy(h)


def say(msg):
    print(msg, flush=True)


# the first shape has T > G at both macro tiles (persistent workgroups run several tiles); ragged M, N and K
SHAPES = [(4352, 4104, 200), (1000, 1032, 520)]


@pytest.mark.parametrize("dtype,dcode,tdt", [("f16", 0, torch.float16), ("bf16", 1, torch.bfloat16)])
@pytest.mark.parametrize("shape", SHAPES)
def test_trace_entries(pg, handle, dtype, dcode, tdt, shape):
    M, N, K = shape
    dev = torch.device("cuda:0")
    A, B = si.operands(M, N, K, dtype, "uniform", workload=13)
    Ad, Bd = A.to(dev), B.to(dev)
    for mode in range(5):
        info = pg.pgemm_query_launch(handle, M, N, K, dcode, mode, 0)
        T, G = info["tiles"], info["grid"]
        say(f"case trace {shape} {dtype} mode {mode} T={T} G={G}")
        C0 = torch.full((M, N), float("nan"), dtype=tdt, device=dev)
        pg.pgemm_run(handle, Ad, Bd, C0, M, N, K, dcode, mode, 0)
        C1 = torch.full((M, N), float("nan"), dtype=tdt, device=dev)
        tr = torch.full((4 * T,), -7, dtype=torch.int64, device=dev)
        own = torch.full((T,), -7, dtype=torch.int32, device=dev)
        vis = torch.zeros(T, dtype=torch.int32, device=dev)
        pg.pgemm_set_tile_trace(handle, tr)
        pg.pgemm_set_owner_log(handle, own)
        pg.pgemm_set_tile_counter(handle, vis)
        try:
            pg.pgemm_run(handle, Ad, Bd, C1, M, N, K, dcode, mode, 0)
            torch.cuda.synchronize()
        finally:
            pg.pgemm_set_tile_trace(handle, None)
            pg.pgemm_set_owner_log(handle, None)
            pg.pgemm_set_tile_counter(handle, None)
        assert np.array_equal(si.bits(C0.cpu()), si.bits(C1.cpu())), mode
        assert np.array_equal(vis.cpu().numpy(), np.ones(T, np.int32)), mode
        t = tr.view(T, 4).cpu().numpy()
        wg, xcd, start, end = t[:, 0], t[:, 1], t[:, 2], t[:, 3]
        assert np.array_equal(wg, own.cpu().numpy().astype(np.int64)), mode
        assert ((xcd >= 0) & (xcd < 8)).all(), mode
        assert (start > 0).all() and (start <= end).all(), mode
        if mode == 4:
            assert (wg < G).all()
        else:
            assert ((wg >= 0) & (wg < G)).all(), mode
        # per workgroup: back-to-back tiles (the stream-K whole-wave and tail launches and
        # the fix-up are separate grids, so only the whole-wave tiles are chained there)
        chained = np.ones(T, bool)
        if mode == 4:
            sk = pg.pgemm_query_streamk(handle, M, N, K, dcode, 0)
            chained = np.arange(T) < sk["whole_tiles"]
        for w in np.unique(wg[chained]):
            idx = np.flatnonzero(chained & (wg == w))
            idx = idx[np.argsort(start[idx], kind="stable")]
            assert np.array_equal(start[idx[1:]], end[idx[:-1]]), (mode, w)
            if mode in (1, 4):
                assert np.array_equal(idx, np.arange(w, w + G * len(idx), G)[:len(idx)]), (mode, w)


def test_short_trace_is_rejected_before_launch(pg, handle):
    dev = torch.device("cuda:0")
    M = N = 1024
    K = 64
    A = torch.zeros(M, K, dtype=torch.float16, device=dev)
    B = torch.zeros(K, N, dtype=torch.float16, device=dev)
    C = torch.full((M, N), 3.0, dtype=torch.float16, device=dev)
    T = pg.pgemm_query_launch(handle, M, N, K, 0, 1, 0)["tiles"]
    tr = torch.zeros(4 * (T - 1), dtype=torch.int64, device=dev)
    pg.pgemm_set_tile_trace(handle, tr)
    try:
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_run(handle, A, B, C, M, N, K, 0, 1, 0)
        assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    finally:
        pg.pgemm_set_tile_trace(handle, None)
    torch.cuda.synchronize()
    assert (C.cpu() == 3.0).all()  # nothing ran
    assert (tr.cpu() == 0).all()


def test_workgroups_dispatch_round_robin_over_xcds(pg):
    """Diagnostic, not a correctness gate: the XCD-aware tile order is meant for workgroups
    dealt round-robin over the 8 XCDs of a whole MI355X (workgroups w and w + 8 share an
    XCD; within a launch the XCD is (w + r) mod 8 for one rotation r). C never depends on
    it (test_xcd_remap_settings_give_the_same_bits is the gate), only the L2 traffic the
    remap saves does. The test checks that the trace's XCD ids are valid and reports the
    fraction of tiles that follow the round-robin rule, with a warning when any does not."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("not a whole 256-CU device")
    dev = torch.device("cuda:0")
    M = N = 8192
    K = 256
    A = torch.zeros(M, K, dtype=torch.float16, device=dev)
    B = torch.zeros(K, N, dtype=torch.float16, device=dev)
    C = torch.empty(M, N, dtype=torch.float16, device=dev)
    h = pg.pgemm_create(0)
    try:
        for mode in (0, 1, 2):
            T = pg.pgemm_query_launch(h, M, N, K, 0, mode, 0)["tiles"]
            tr = torch.zeros(4 * T, dtype=torch.int64, device=dev)
            pg.pgemm_set_tile_trace(h, tr)
            try:
                pg.pgemm_run(h, A, B, C, M, N, K, 0, mode, 0)
                torch.cuda.synchronize()
            finally:
                pg.pgemm_set_tile_trace(h, None)
            t = tr.view(T, 4).cpu().numpy()
            assert ((t[:, 1] >= 0) & (t[:, 1] < 8)).all(), mode
            rot = (t[:, 1] - t[:, 0]) % 8
            frac = float(np.bincount(rot, minlength=8).max()) / T
            say(f"case xcd dispatch mode {mode}: fraction of tiles on XCD (w + r) mod 8: {frac:.4f}")
            if frac < 1.0:
                warnings.warn(f"mode {mode}: only {frac:.4f} of the tiles follow the round-robin XCD rule; "
                              "the XCD-aware tile order then saves less L2 traffic (C is unaffected)")
    finally:
        pg.pgemm_destroy(h)
