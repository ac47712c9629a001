"""GPU parity: every scheduling mode x dtype against the CPU oracle, through the C ABI.

Checks, per case (see the oracle's header for what is computed):
* normwise error ||C - C_ref||_F / ||C_ref||_F <= 2e-3 (fp16/bf16 out) or
  <= 1e-2 (fp8 in, bf16 out);
* small-integer inputs: bit-exact against the oracle's value rounded to the
  output type (every partial sum is an integer below 2^24, exact in fp32 in
  any order);
* tile-visit counter: every output tile written exactly once;
* C bitwise identical across the four tile-scheduling modes (one tile
  body); the stream-K mode, which adds split tiles' partial sums, is held
  to the oracle bound (and to bit-exactness on small integers) instead.

Every case runs with each macro-tile configuration of the fast kernel
(256 x 256 and 128 x 128), selected explicitly through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

DT = {"f16": 0, "bf16": 1, "e4m3fn": 2}
OUT = {"f16": ("f16", torch.float16), "bf16": ("bf16", torch.bfloat16), "e4m3fn": ("bf16", torch.bfloat16)}
TOL = {"f16": 2e-3, "bf16": 2e-3, "e4m3fn": 1e-2}
MODES = [0, 1, 2, 3, 4]  # non-persistent, static, dynamic, cancel-and-reuse, stream-K
SAME_BITS = [0, 1, 2, 3]  # modes that run every tile whole: C bitwise identical
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


def run(pg, h, A, B, dtype, mode, grid_multiple=0, visits=True):
    """Run C = A @ B on the GPU; returns (C bits, visits array or None, launch info)."""
    M, K = A.shape
    N = B.shape[1]
    dev = torch.device("cuda:0")
    Ad, Bd = A.to(dev), B.to(dev)
    C = torch.full((M, N), float("nan"), dtype=OUT[dtype][1], device=dev)
    info = pg.pgemm_query_launch(h, M, N, K, DT[dtype], mode, grid_multiple)
    v = None
    if visits and M and N and K:
        v = torch.zeros(max(info["tiles"], 1), dtype=torch.int32, device=dev)
        pg.pgemm_set_tile_counter(h, v)
    try:
        pg.pgemm_run(h, Ad, Bd, C, M, N, K, DT[dtype], mode, grid_multiple)
        torch.cuda.synchronize()
    finally:
        pg.pgemm_set_tile_counter(h, None)
    return si.bits(C.cpu()), (v.cpu().numpy() if v is not None else None), info


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
def test_workload_256_all_modes(pg, handle, dtype):
    """fp16 256^3 uniform[-1,1] (seeds 2, 3) and the same shape in bf16 / fp8."""
    A, B = si.operands(256, 256, 256, dtype, "uniform", workload=1)
    ref = oracle.gemm(si.bits(A), si.bits(B), dtype)
    outs = []
    for mode in MODES:
        say(f"case 256^3 {dtype} mode {mode}")
        c, v, info = run(pg, handle, A, B, dtype, mode)
        err = oracle.normwise_error(c, OUT[dtype][0], ref)
        assert err <= TOL[dtype], (mode, err)
        assert info["fast_path"] == 1 and info["tiles"] == (256 // info["bm"]) * (256 // info["bn"])
        assert np.array_equal(v, np.ones_like(v)), v
        if mode in SAME_BITS:
            outs.append(c)
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


SHAPES_INT = [(1, 1, 1), (7, 9, 5), (256, 256, 64), (300, 520, 200), (513, 264, 136), (64, 2048, 640),
              (1, 784, 48), (259, 16, 1040),
              # odd and edge sizes: 17, 33, 127, 129, 255, 257 (unaligned: generic body), and the
              # tail set's 4000 = 15*256 + 160 and 8200 = 32*256 + 8 in either dimension
              (17, 33, 127), (129, 257, 255), (4000, 4000, 48), (8200, 264, 32), (264, 8200, 48)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
@pytest.mark.parametrize("shape", SHAPES_INT)
def test_small_integers_bit_exact(pg, handle, dtype, shape):
    M, N, K = shape
    A, B = si.operands(M, N, K, dtype, "small_int", workload=7)
    ref = oracle.gemm(si.bits(A), si.bits(B), dtype)
    want = oracle.round_to(ref, OUT[dtype][0])
    for mode in MODES:
        say(f"case small-int {shape} {dtype} mode {mode}")
        c, v, info = run(pg, handle, A, B, dtype, mode)
        assert np.array_equal(c, want), (mode, np.argwhere(c != want)[:5])
        assert np.array_equal(v[:info["tiles"]], np.ones(info["tiles"], np.int32))


SHAPES_RAND = [(1000, 1032, 520), (777, 333, 129), (512, 768, 1024), (257, 1024, 4096)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
@pytest.mark.parametrize("shape", SHAPES_RAND)
def test_uniform_parity(pg, handle, dtype, shape):
    M, N, K = shape
    A, B = si.operands(M, N, K, dtype, "uniform", workload=11)
    ref = oracle.gemm(si.bits(A), si.bits(B), dtype)
    outs = []
    for mode in MODES:
        say(f"case uniform {shape} {dtype} mode {mode}")
        c, v, info = run(pg, handle, A, B, dtype, mode)
        err = oracle.normwise_error(c, OUT[dtype][0], ref)
        assert err <= TOL[dtype], (mode, err)
        assert np.array_equal(v[:info["tiles"]], np.ones(info["tiles"], np.int32))
        if mode in SAME_BITS:
            outs.append(c)
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


def test_brute_force_tiny(pg, handle):
    """Every (M, N, K) in {1..9}^3, every mode, fp16 small integers: bit-exact."""
    for M in range(1, 10):
        for N in range(1, 10):
            for K in range(1, 10):
                A, B = si.operands(M, N, K, "f16", "small_int", workload=M * 100 + N * 10 + K)
                want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
                for mode in MODES:
                    c, v, _ = run(pg, handle, A, B, "f16", mode)
                    assert np.array_equal(c, want), (M, N, K, mode)
                    assert v[0] == 1


def test_static_owner_map_and_dynamic_counter(pg, handle):
    """Static: owner[t] = t mod G (deterministic mapping). Dynamic and
    cancel-and-reuse: every tile once, the work counter back at 0 after each
    launch, also back to back and interleaved with each other."""
    dev = torch.device("cuda:0")
    M, N, K = 8192, 4096, 64  # 512 tiles of 256 x 256 or 2048 of 128 x 128
    A, B = si.operands(M, N, K, "f16", "small_int", workload=3)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
    Ad, Bd = A.to(dev), B.to(dev)
    for gm in (1, 2, 3):
        info = pg.pgemm_query_launch(handle, M, N, K, 0, 1, gm)
        T, G = info["tiles"], info["grid"]
        owner = torch.full((T,), -1, dtype=torch.int32, device=dev)
        pg.pgemm_set_owner_log(handle, owner)
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
        say(f"case owner map static gm={gm} T={T} G={G}")
        pg.pgemm_run(handle, Ad, Bd, C, M, N, K, 0, 1, gm)
        torch.cuda.synchronize()
        pg.pgemm_set_owner_log(handle, None)
        assert np.array_equal(owner.cpu().numpy(), np.arange(T) % G)
        assert np.array_equal(si.bits(C.cpu()), want)
    T = pg.pgemm_query_launch(handle, M, N, K, 0, 2, 0)["tiles"]
    visits = torch.zeros(T, dtype=torch.int32, device=dev)
    pg.pgemm_set_tile_counter(handle, visits)
    try:
        for rep in range(4):
            C = torch.empty((M, N), dtype=torch.float16, device=dev)
            say(f"case dynamic / cancel back-to-back rep {rep}")
            pg.pgemm_run(handle, Ad, Bd, C, M, N, K, 0, 2, 1)
            pg.pgemm_run(handle, Ad, Bd, C, M, N, K, 0, 3, 0)
            pg.pgemm_run(handle, Ad, Bd, C, M, N, K, 0, 2, 0)
            torch.cuda.synchronize()
            assert pg.pgemm_read_work_counter(handle) == 0
            assert np.array_equal(si.bits(C.cpu()), want)
        assert np.array_equal(visits.cpu().numpy(), np.full(T, 12, np.int32))
    finally:
        pg.pgemm_set_tile_counter(handle, None)
    # cancel-and-reuse: grid = T, every tile's owner is a workgroup of that grid
    info = pg.pgemm_query_launch(handle, M, N, K, 0, 3, 0)
    assert info["grid"] == info["tiles"] == T
    owner = torch.full((T,), -1, dtype=torch.int32, device=dev)
    pg.pgemm_set_owner_log(handle, owner)
    try:
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
        pg.pgemm_run(handle, Ad, Bd, C, M, N, K, 0, 3, 0)
        torch.cuda.synchronize()
    finally:
        pg.pgemm_set_owner_log(handle, None)
    o = owner.cpu().numpy()
    assert o.min() >= 0 and o.max() < T
    assert np.array_equal(si.bits(C.cpu()), want)


def test_xcd_remap_settings_give_the_same_bits(pg, handle):
    """The XCD remap (off, on, automatic) only moves tiles between
    workgroups: on a problem with more tiles than CUs (so the automatic
    setting turns it on) C is bit-exact against the oracle and every tile is
    written once, in every tile-scheduling mode."""
    M, N, K = 4352, 4352, 64  # 289 tiles of 256 x 256, 1156 of 128 x 128
    A, B = si.operands(M, N, K, "f16", "small_int", workload=3)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        for remap in (0, 1, None):
            pg.pgemm_set_tile_order(handle, 4, remap)
            for mode in SAME_BITS:
                say(f"case xcd remap {remap} mode {mode} {M}x{N}x{K}")
                c, v, info = run(pg, handle, A, B, "f16", mode)
                assert info["tiles"] > cus
                assert np.array_equal(c, want), (remap, mode)
                assert (v == 1).all(), (remap, mode)
    finally:
        pg.pgemm_set_tile_order(handle, 4, None)


def test_degenerate_sizes(pg, handle):
    dev = torch.device("cuda:0")
    A = torch.ones((5, 0), dtype=torch.float16, device=dev)
    B = torch.ones((0, 7), dtype=torch.float16, device=dev)
    C = torch.full((5, 7), 3.0, dtype=torch.float16, device=dev)
    for mode in MODES:
        pg.pgemm_run(handle, A, B, C, 5, 7, 0, 0, mode, 0)  # K = 0: an empty sum
        torch.cuda.synchronize()
        assert torch.all(C == 0)
        C.fill_(3.0)
    pg.pgemm_run(handle, 0, 0, 0, 0, 7, 9, 0, 1, 0)  # M = 0: nothing to do
    pg.pgemm_run(handle, 0, 0, 0, 5, 0, 9, 0, 1, 0)


def test_invalid_arguments(pg, handle):
    dev = torch.device("cuda:0")
    A = torch.ones((4, 8), dtype=torch.float16, device=dev)
    with pytest.raises(pg.PgemmError) as e:
        pg.pgemm_run(handle, A, A, A, -1, 8, 8, 0, 1, 0)
    assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    with pytest.raises(pg.PgemmError):
        pg.pgemm_run(handle, A, A, A, 4, 8, 8, 7, 1, 0)
    with pytest.raises(pg.PgemmError):
        pg.pgemm_run(handle, A, A, A, 4, 8, 8, 0, 5, 0)
    with pytest.raises(pg.PgemmError):
        pg.pgemm_run(handle, 0, A, A, 4, 8, 8, 0, 1, 0)
    small = torch.zeros(1, dtype=torch.int32, device=dev)
    pg.pgemm_set_tile_counter(handle, small)
    try:
        with pytest.raises(pg.PgemmError):
            big = torch.zeros((600, 600), dtype=torch.float16, device=dev)
            pg.pgemm_run(handle, big, big, big, 600, 600, 600, 0, 1, 0)  # 9 tiles > 1 counter
    finally:
        pg.pgemm_set_tile_counter(handle, None)


def test_modes_while_cus_are_held(pg, handle):
    """Every mode stays exact while another kernel holds half the CUs (its
    workgroups then start late or wait for CUs): bit-exact small-integer C,
    every tile written once, the work counter back at 0."""
    dev = torch.device("cuda:0")
    M, N, K = 2048, 2048, 512
    A, B = si.operands(M, N, K, "f16", "small_int", workload=9)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
    Ad, Bd = A.to(dev), B.to(dev)
    side = torch.cuda.Stream(device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for mode in MODES:
        T = pg.pgemm_query_launch(handle, M, N, K, 0, mode, 0)["tiles"]
        visits = torch.zeros(T, dtype=torch.int32, device=dev)
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        say(f"case held CUs mode {mode} T={T}")
        pg.pgemm_set_tile_counter(handle, visits)
        try:
            pg.pgemm_hold_cus(side, 0, cus // 2, 2000)
            pg.pgemm_run(handle, Ad, Bd, C, M, N, K, 0, mode, 0)
            torch.cuda.synchronize()
        finally:
            pg.pgemm_set_tile_counter(handle, None)
        assert bool(torch.all(visits == 1)), mode
        assert np.array_equal(si.bits(C.cpu()), want), mode
        assert pg.pgemm_read_work_counter(handle) == 0


def test_producer_wave_body_launch_report(pg):
    """The producer-wave mainloop runs the 256 x 128 tile body (body 3) in the four
    tile-sequence modes, at every size the fast kernel takes, and leaves stream-K on the
    lockstep 256 x 256 body (body 1), with the 256-row tile chosen."""
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(h, pg.PGEMM_TILE_256)
        pg.pgemm_set_mainloop(h, pg.PGEMM_MAINLOOP_PRODUCER)
        for dcode in (0, 1, 2):
            for (M, N, K) in [(256, 256, 64), (8192, 8192, 8192), (1000, 1040, 528)]:  # fast-kernel sizes for every dtype
                for mode in (0, 1, 2, 3):
                    info = pg.pgemm_query_launch(h, M, N, K, dcode, mode, 0)
                    assert (info["body"], info["bm"], info["bn"]) == (3, 256, 128), (dcode, M, mode, info)
                    assert info["tiles"] == -(-M // 256) * -(-N // 128)
                info = pg.pgemm_query_launch(h, M, N, K, dcode, 4, 0)
                assert (info["body"], info["bm"], info["bn"]) == (1, 256, 256), (dcode, M, info)
        with pytest.raises(pg.PgemmError):
            pg.pgemm_set_mainloop(h, 4)
    finally:
        pg.pgemm_destroy(h)


# (tile config, mainloop, M, N, K): 48 tiles of 128^2, where stream-K splits each in two (a
# fix-up node too); and 256-row tiles with a k-loop long enough for the ping-pong body
# (stream-K: a ping-pong whole-wave launch, a lockstep tail and a fix-up) and the producer body
GRAPH_CASES = {"t128": (2, 0, 1024, 768, 1024), "t256_pingpong": (1, 2, 1280, 1024, 2048),
               "t256x128_producer": (1, 3, 1280, 1024, 2048)}


@pytest.mark.parametrize("case", sorted(GRAPH_CASES))
def test_graph_capture_and_replay(pg, case):
    """pgemm_run is capture-safe: no memsets, and the claiming modes' work
    counter resets itself inside the kernel. A HIP graph holding one launch per
    scheduling mode is replayed several times with eager work in between;
    every replay's C is bit-exact and the counter reads 0 after each."""
    tile, mainloop, M, N, K = GRAPH_CASES[case]
    dev = torch.device("cuda:0")
    A, B = si.operands(M, N, K, "f16", "small_int", workload=13)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "f16"), "f16")
    Ad, Bd = A.to(dev), B.to(dev)
    Cs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in MODES]
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(h, tile)
        pg.pgemm_set_mainloop(h, mainloop)
        for C, mode in zip(Cs, MODES):  # eager runs first: any stream-K workspace exists before capture
            pg.pgemm_run(h, Ad, Bd, C, M, N, K, 0, mode, 0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            pg.pgemm_set_stream(h, torch.cuda.current_stream())
            for C, mode in zip(Cs, MODES):
                pg.pgemm_run(h, Ad, Bd, C, M, N, K, 0, mode, 0)
        pg.pgemm_set_stream(h, torch.cuda.current_stream())
        for rep in range(4):
            for C in Cs:
                C.fill_(float("nan"))  # eager work between replays
            say(f"case graph replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            for C, mode in zip(Cs, MODES):
                assert np.array_equal(si.bits(C.cpu()), want), (rep, mode)
            assert pg.pgemm_read_work_counter(h) == 0
    finally:
        pg.pgemm_destroy(h)


def test_size_limits_are_rejected_before_any_launch(pg):
    """The fast kernel's buffer offsets are 32-bit: a tile's A rows (BM x K
    elements) and a k-step's B rows (BK x N elements) must span < 2^31 bytes.
    The planner refuses larger problems with PGEMM_ERR_UNSUPPORTED (checked
    through the launch query, which plans exactly as pgemm_run does but
    launches nothing), and accepts the largest ones inside the limits."""
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(h, pg.PGEMM_TILE_256)
        k_max = (1 << 31) // (256 * 2)  # 256 rows of fp16 A
        ok = pg.pgemm_query_launch(h, 256, 256, k_max - 8, 0, 1, 0)
        assert ok["fast_path"] == 1
        for mode in (0, 1, 2, 3, 4):
            with pytest.raises(pg.PgemmError) as e:
                pg.pgemm_query_launch(h, 256, 256, k_max, 0, mode, 0)
            assert e.value.status == pg.PGEMM_ERR_UNSUPPORTED, mode
        n_max = (1 << 31) // (64 * 2)  # 64 k-rows of fp16 B
        pg.pgemm_query_launch(h, 256, n_max - 8, 256, 0, 1, 0)
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_query_launch(h, 256, n_max, 256, 0, 1, 0)
        assert e.value.status == pg.PGEMM_ERR_UNSUPPORTED
        with pytest.raises(pg.PgemmError) as e:  # sizes beyond int32
            pg.pgemm_query_launch(h, 1 << 31, 256, 256, 0, 1, 0)
        assert e.value.status == pg.PGEMM_ERR_UNSUPPORTED
    finally:
        pg.pgemm_destroy(h)


def test_two_handles_on_two_streams_and_reruns(pg):
    """Two handles, each bound to its own stream, run the claiming modes at the same time:
    each handle's work counter serves only its own launches (every tile once per launch,
    both counters back at 0), and ten back-to-back reruns per handle give the same bits."""
    dev = torch.device("cuda:0")
    probs = [(1000, 1032, 520, "f16"), (777, 1024, 264, "bf16")]
    hs, streams, ins = [], [], []
    for i, (M, N, K, dt) in enumerate(probs):
        h = pg.pgemm_create(0)
        st = torch.cuda.Stream()
        pg.pgemm_set_stream(h, st)
        pg.pgemm_set_tile_config(h, 2)  # 128 x 128: several tiles per persistent workgroup
        A, B = si.operands(M, N, K, dt, "small_int", workload=30 + i)
        ins.append((A.to(dev), B.to(dev), oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), dt), dt)))
        hs.append(h)
        streams.append(st)
    torch.cuda.synchronize()
    try:
        for mode in (2, 3):  # dynamic, cancel-and-reuse
            say(f"case two handles mode {mode}")
            outs, vis = [], []
            for (M, N, K, dt), h, st, (A, B, _) in zip(probs, hs, streams, ins):
                T = pg.pgemm_query_launch(h, M, N, K, DT[dt], mode, 0)["tiles"]
                vis.append(torch.zeros((10, T), dtype=torch.int32, device=dev))
                outs.append([torch.empty((M, N), dtype=OUT[dt][1], device=dev) for _ in range(10)])
            # interleave the two handles' launches on their two streams
            for r in range(10):
                for i, ((M, N, K, dt), h) in enumerate(zip(probs, hs)):
                    A, B, _ = ins[i]
                    pg.pgemm_set_tile_counter(hs[i], vis[i][r])
                    pg.pgemm_run(h, A, B, outs[i][r], M, N, K, DT[dt], mode, 0)
            torch.cuda.synchronize()
            for i, ((M, N, K, dt), h) in enumerate(zip(probs, hs)):
                pg.pgemm_set_tile_counter(h, None)
                assert (vis[i].cpu() == 1).all(), (mode, i)
                assert pg.pgemm_read_work_counter(h) == 0
                want = ins[i][2]
                for r in range(10):
                    assert np.array_equal(si.bits(outs[i][r].cpu()), want), (mode, i, r)
    finally:
        for h in hs:
            pg.pgemm_destroy(h)
