"""GPU parity of per-tensor e4m3 scales (pgemm_set_fp8_scales), through the C ABI.

The oracle applies the scales in double (C = sA * sB * sum of decoded
products). Checks, per macro tile and scheduling mode (stream-K splits and
the generic body included):
* power-of-two scales on small-integer inputs: bit-exact (the fp32 sum, the
  fp32 product of the scales and their product are all exact);
* general scales on uniform inputs: within the fp8 normwise bound;
* the default scales leave C bitwise unchanged, and 16-bit dtypes ignore them;
* non-finite scales are rejected.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

# (tile config, mainloop): the 256 x 256 tile with lockstep waves and in ping-pong, the 256 x 128
# tile of the producer-wave body (stream-K keeps the lockstep 256 x 256 body), and 128 x 128
TILES = {"t256_lockstep": (1, 1), "t256_pingpong": (1, 2), "t256x128_producer": (1, 3), "t128": (2, 0)}
F8 = 2


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
    pg.pgemm_set_fp8_scales(h, 1.0, 1.0)
    pg.pgemm_destroy(h)


def say(msg):
    print(msg, flush=True)


def run(pg, h, A, B, M, N, K, dcode, mode, out=torch.bfloat16):
    dev = torch.device("cuda:0")
    C = torch.full((M, N), float("nan"), dtype=out, device=dev)
    pg.pgemm_run(h, A.to(dev), B.to(dev), C, M, N, K, dcode, mode, 0)
    torch.cuda.synchronize()
    return si.bits(C.cpu())


# fast path with ragged edges, a long K (stream-K splits at the 128 tile), and an unaligned shape
SHAPES = [(1000, 1008, 528), (256, 256, 8192), (300, 264, 136)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scales", [(0.5, 4.0), (0.25, 0.125), (-2.0, 0.5)])
def test_power_of_two_scales_bit_exact(pg, handle, shape, scales):
    M, N, K = shape
    sa, sb = scales
    A, B = si.operands(M, N, K, "e4m3fn", "small_int", workload=50)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "e4m3fn", scale_a=sa, scale_b=sb), "bf16")
    pg.pgemm_set_fp8_scales(handle, sa, sb)
    try:
        for mode in range(5):
            say(f"case fp8 scales {scales} {shape} mode {mode}")
            c = run(pg, handle, A, B, M, N, K, F8, mode)
            assert np.array_equal(c, want), (mode, np.argwhere(c != want)[:5])
    finally:
        pg.pgemm_set_fp8_scales(handle, 1.0, 1.0)


def test_general_scales_within_bound(pg, handle):
    M, N, K = 1000, 1008, 528
    sa, sb = 0.37, 1.9
    A, B = si.operands(M, N, K, "e4m3fn", "uniform", workload=51)
    ref = oracle.gemm(si.bits(A), si.bits(B), "e4m3fn", scale_a=sa, scale_b=sb)
    pg.pgemm_set_fp8_scales(handle, sa, sb)
    try:
        for mode in range(5):
            say(f"case fp8 general scales mode {mode}")
            c = run(pg, handle, A, B, M, N, K, F8, mode)
            assert oracle.normwise_error(c, "bf16", ref) <= 1e-2, mode
    finally:
        pg.pgemm_set_fp8_scales(handle, 1.0, 1.0)


def test_default_scales_and_16bit_dtypes_unchanged(pg, handle):
    M, N, K = 512, 528, 272
    A8, B8 = si.operands(M, N, K, "e4m3fn", "uniform", workload=52)
    A16, B16 = si.operands(M, N, K, "f16", "uniform", workload=52)
    fresh = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(fresh, 1)
        pg.pgemm_set_tile_config(handle, 1)
        c8_fresh = run(pg, fresh, A8, B8, M, N, K, F8, 1)
        pg.pgemm_set_fp8_scales(handle, 1.0, 1.0)
        assert np.array_equal(run(pg, handle, A8, B8, M, N, K, F8, 1), c8_fresh)
        c16_fresh = run(pg, fresh, A16, B16, M, N, K, 0, 1, torch.float16)
        pg.pgemm_set_fp8_scales(handle, 8.0, 0.25)
        assert np.array_equal(run(pg, handle, A16, B16, M, N, K, 0, 1, torch.float16), c16_fresh)
    finally:
        pg.pgemm_set_fp8_scales(handle, 1.0, 1.0)
        pg.pgemm_destroy(fresh)


def test_non_finite_scales_rejected(pg, handle):
    for sa, sb in [(math.inf, 1.0), (1.0, math.nan), (3e38, 3e38)]:
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_set_fp8_scales(handle, sa, sb)
        assert e.value.status == pg.PGEMM_ERR_INVALID_ARG


def test_scales_with_nk_layout_and_trace(pg, handle):
    """The features together: e4m3 with B stored N x K, power-of-two scales and the tile
    trace (its own kernel instantiation) -- bit-exact on small integers in every mode,
    and every tile traced once with start <= end."""
    M, N, K = 1000, 1008, 4000  # ragged edges; long K (stream-K splits at the 128 tile)
    sa, sb = 0.5, 2.0
    A, B = si.operands(M, N, K, "e4m3fn", "small_int", workload=53)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), "e4m3fn", scale_a=sa, scale_b=sb), "bf16")
    Bt = B.t().contiguous()
    dev = torch.device("cuda:0")
    pg.pgemm_set_fp8_scales(handle, sa, sb)
    pg.pgemm_set_b_layout(handle, pg.PGEMM_B_NK)
    try:
        for mode in range(5):
            T = pg.pgemm_query_launch(handle, M, N, K, F8, mode, 0)["tiles"]
            tr = torch.zeros(4 * T, dtype=torch.int64, device=dev)
            pg.pgemm_set_tile_trace(handle, tr)
            try:
                say(f"case fp8 NK scales trace mode {mode} T={T}")
                c = run(pg, handle, A, Bt, M, N, K, F8, mode)
            finally:
                pg.pgemm_set_tile_trace(handle, None)
            assert np.array_equal(c, want), (mode, np.argwhere(c != want)[:5])
            t = tr.view(T, 4).cpu().numpy()
            assert (t[:, 2] > 0).all() and (t[:, 2] <= t[:, 3]).all(), mode
    finally:
        pg.pgemm_set_fp8_scales(handle, 1.0, 1.0)
        pg.pgemm_set_b_layout(handle, pg.PGEMM_B_KN)
