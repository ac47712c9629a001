"""GPU checks of pgemm_run_ld (operands that are row-major views with leading dimensions).

Per dtype, macro tile, B layout and scheduling mode:
* A, B and C are windows inside larger allocations: C's window is bitwise
  equal to pgemm_run on contiguous copies, and the padding around it is
  untouched;
* unaligned leading dimensions take the generic body and stay bit-exact on
  small integers against the oracle;
* K = 0 zeroes only C's window; leading dimensions shorter than their rows
  are rejected before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

DT = {"f16": (0, torch.float16), "bf16": (1, torch.bfloat16), "e4m3fn": (2, torch.bfloat16)}
# (tile config, mainloop): the 256 x 256 tile with lockstep waves and in ping-pong, the 256 x 128
# tile of the producer-wave body (stream-K keeps the lockstep 256 x 256 body), and 128 x 128
TILES = {"t256_lockstep": (1, 1), "t256_pingpong": (1, 2), "t256x128_producer": (1, 3), "t128": (2, 0)}
SENT = 5.0  # padding sentinel, exact in fp16 and bf16


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
    pg.pgemm_set_b_layout(h, pg.PGEMM_B_KN)
    pg.pgemm_destroy(h)


def say(msg):
    print(msg, flush=True)


def embed(x, rows, cols, r0, c0, dev):
    """A (rows x cols) buffer holding x at (r0, c0), the rest zeros; returns (buffer, view)."""
    big = torch.zeros((rows, cols), dtype=x.dtype, device=dev)
    big[r0:r0 + x.shape[0], c0:c0 + x.shape[1]] = x.to(dev)
    return big, big[r0:r0 + x.shape[0], c0:c0 + x.shape[1]]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
@pytest.mark.parametrize("nk", [False, True])
def test_views_match_contiguous_runs(pg, handle, dtype, nk):
    dcode, odt = DT[dtype]
    dev = torch.device("cuda:0")
    M, N, K = 1000, 1008, 528
    A, B = si.operands(M, N, K, dtype, "uniform", workload=60)
    Bs = B.t().contiguous() if nk else B  # stored B
    pg.pgemm_set_b_layout(handle, pg.PGEMM_B_NK if nk else pg.PGEMM_B_KN)
    # windows at 16-element offsets inside wider rows (leading dimensions stay 16-byte multiples)
    Abig, Av = embed(A, M + 3, K + 48, 1, 16, dev)
    Bbig, Bv = embed(Bs, Bs.shape[0] + 2, Bs.shape[1] + 32, 2, 16, dev)
    for mode in range(5):
        say(f"case run_ld views {dtype} nk={nk} mode {mode}")
        C0 = torch.empty((M, N), dtype=odt, device=dev)
        pg.pgemm_run(handle, A.to(dev), Bs.to(dev), C0, M, N, K, dcode, mode, 0)
        Cbig = torch.full((M + 4, N + 24), SENT, dtype=odt, device=dev)
        Cv = Cbig[2:2 + M, 8:8 + N]
        pg.pgemm_run_ld(handle, Av, Abig.shape[1], Bv, Bbig.shape[1], Cv, Cbig.shape[1], M, N, K, dcode, mode, 0)
        torch.cuda.synchronize()
        assert np.array_equal(si.bits(Cv.cpu()), si.bits(C0.cpu())), mode
        pad = Cbig.clone()
        pad[2:2 + M, 8:8 + N] = SENT
        assert (pad.cpu() == SENT).all(), mode


@pytest.mark.parametrize("dtype", ["f16", "e4m3fn"])
def test_unaligned_leading_dimensions_take_the_generic_body(pg, handle, dtype):
    dcode, odt = DT[dtype]
    dev = torch.device("cuda:0")
    M, N, K = 300, 264, 144
    A, B = si.operands(M, N, K, dtype, "small_int", workload=61)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), dtype), "f16" if dtype == "f16" else "bf16")
    pg.pgemm_set_b_layout(handle, pg.PGEMM_B_KN)
    Abig, Av = embed(A, M, K + 3, 0, 1, dev)  # odd leading dimension, odd offset
    Bbig, Bv = embed(B, K, N + 5, 0, 3, dev)
    for mode in range(5):
        say(f"case run_ld unaligned {dtype} mode {mode}")
        Cbig = torch.full((M, N + 1), SENT, dtype=odt, device=dev)
        Cv = Cbig[:, 1:]
        pg.pgemm_run_ld(handle, Av, K + 3, Bv, N + 5, Cv, N + 1, M, N, K, dcode, mode, 0)
        torch.cuda.synchronize()
        assert np.array_equal(si.bits(Cv.cpu()), want), mode
        assert (Cbig[:, 0].cpu() == SENT).all()


def test_k0_zeroes_only_the_window_and_bad_strides_are_rejected(pg, handle):
    dev = torch.device("cuda:0")
    M, N = 100, 64
    Cbig = torch.full((M, N + 16), SENT, dtype=torch.float16, device=dev)
    pg.pgemm_set_b_layout(handle, pg.PGEMM_B_KN)
    pg.pgemm_run_ld(handle, 0, 0, 0, 0, Cbig[:, 8:8 + N], N + 16, M, N, 0, 0, 1, 0)
    torch.cuda.synchronize()
    c = Cbig.cpu()
    assert (c[:, 8:8 + N] == 0).all() and (c[:, :8] == SENT).all() and (c[:, 8 + N:] == SENT).all()
    A = torch.zeros((M, 32), dtype=torch.float16, device=dev)
    B = torch.zeros((32, N), dtype=torch.float16, device=dev)
    for lda, ldb, ldc in [(31, N, N), (32, N - 1, N), (32, N, N - 1), (2 ** 31, N, N)]:
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_run_ld(handle, A, lda, B, ldb, Cbig, ldc, M, N, 32, 0, 1, 0)
        assert e.value.status == pg.PGEMM_ERR_INVALID_ARG, (lda, ldb, ldc)
    torch.cuda.synchronize()
    assert (Cbig.cpu()[:, :8] == SENT).all()
