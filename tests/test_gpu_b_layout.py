"""GPU parity of B stored as N x K (pgemm_set_b_layout(PGEMM_B_NK)), through the C ABI.

The oracle always takes B as K x N; the GPU gets the same values stored
transposed. Checks, per dtype, macro tile and scheduling mode:
* small-integer inputs: bit-exact against the oracle (every partial sum is an
  integer below 2^24, exact in fp32 in any order);
* uniform inputs: C bitwise equal to the K x N layout's C (both layouts feed
  the MFMAs the same operands in the same order) and within the normwise
  bound of the oracle;
* the visit counter reads all ones;
* unaligned sizes take the generic body, which reads B in either layout.
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
def handles(pg, request):
    kn, nk = pg.pgemm_create(0), pg.pgemm_create(0)
    for h in (kn, nk):
        pg.pgemm_set_tile_config(h, TILES[request.param][0])
    pg.pgemm_set_mainloop(h, TILES[request.param][1])
    pg.pgemm_set_b_layout(nk, pg.PGEMM_B_NK)
    yield kn, nk
    pg.pgemm_destroy(kn)
    pg.pgemm_destroy(nk)


def say(msg):
    print(msg, flush=True)


def run(pg, h, A, Bmat, M, N, K, dtype, mode):
    dev = torch.device("cuda:0")
    C = torch.full((M, N), float("nan"), dtype=OUT[dtype][1], device=dev)
    T = pg.pgemm_query_launch(h, M, N, K, DT[dtype], mode, 0)["tiles"]
    v = torch.zeros(max(T, 1), dtype=torch.int32, device=dev)
    pg.pgemm_set_tile_counter(h, v)
    try:
        pg.pgemm_run(h, A.to(dev), Bmat.to(dev), C, M, N, K, DT[dtype], mode, 0)
        torch.cuda.synchronize()
    finally:
        pg.pgemm_set_tile_counter(h, None)
    assert (v.cpu()[:T] == 1).all()
    return si.bits(C.cpu())


# fast path (K and N multiples of 16 elements, ragged M/N/K edges, a K tail) and unaligned sizes
SHAPES = [(1000, 1008, 528), (256, 512, 2048), (300, 264, 144), (777, 333, 129), (33, 17, 9)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
@pytest.mark.parametrize("shape", SHAPES)
def test_nk_layout_small_integers_bit_exact(pg, handles, dtype, shape):
    kn, nk = handles
    M, N, K = shape
    A, B = si.operands(M, N, K, dtype, "small_int", workload=40)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), dtype), OUT[dtype][0])
    Bt = B.t().contiguous()
    for mode in range(5):
        say(f"case B NK small-int {shape} {dtype} mode {mode}")
        c = run(pg, nk, A, Bt, M, N, K, dtype, mode)
        assert np.array_equal(c, want), (mode, np.argwhere(c != want)[:5])


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
@pytest.mark.parametrize("shape", [(1000, 1008, 528), (4000, 1024, 4000)])
def test_nk_layout_uniform_equals_kn_layout(pg, handles, dtype, shape):
    kn, nk = handles
    M, N, K = shape
    A, B = si.operands(M, N, K, dtype, "uniform", workload=41)
    rows = list(range(0, M, 97)) + [M - 1]
    ref = oracle.gemm(si.bits(A), si.bits(B), dtype, rows=rows)
    Bt = B.t().contiguous()
    for mode in range(5):
        say(f"case B NK uniform {shape} {dtype} mode {mode}")
        c_kn = run(pg, kn, A, B, M, N, K, dtype, mode)
        c_nk = run(pg, nk, A, Bt, M, N, K, dtype, mode)
        assert np.array_equal(c_kn, c_nk), mode
        err = oracle.normwise_error(c_nk[rows], OUT[dtype][0], ref)
        assert err <= TOL[dtype], (mode, err)


def test_b_layout_rejects_unknown_values(pg):
    h = pg.pgemm_create(0)
    try:
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_set_b_layout(h, 2)
        assert e.value.status == pg.PGEMM_ERR_INVALID_ARG
    finally:
        pg.pgemm_destroy(h)
