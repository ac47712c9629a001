"""GPU check of the watchdog wait (pgemm_wait), through the C ABI.

The long-running work is the CU-holding benchmark kernel, which idles for a
set time on the device's constant-rate clock and then ends normally: the
time-out is forced from the host by a deadline shorter than that time."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_macro_amd as pg
    return pg


def test_wait_times_out_then_completes(pg):
    stream = torch.cuda.Stream()
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_stream(h, stream)
        pg.pgemm_wait(h, 0)  # nothing enqueued: idle at once
        print("case watchdog: 8 CUs held for 200 ms, 5 ms deadline", flush=True)
        pg.pgemm_hold_cus(stream, 0, 8, 200_000)
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_wait(h, 5)
        assert e.value.status == pg.PGEMM_ERR_TIMEOUT
        assert "still busy" in pg.pgemm_last_error(h)
        pg.pgemm_wait(h, 20_000)  # the hold ends by itself
        # a GEMM on the same stream, waited for the same way
        M = N = K = 512
        A = torch.ones(M, K, dtype=torch.float16, device="cuda:0")
        B = torch.ones(K, N, dtype=torch.float16, device="cuda:0")
        C = torch.zeros(M, N, dtype=torch.float16, device="cuda:0")
        torch.cuda.synchronize()
        pg.pgemm_run(h, A, B, C, M, N, K, pg.PGEMM_F16, pg.PGEMM_SCHED_STATIC, 0)
        pg.pgemm_wait(h, 20_000)
        assert (C.cpu() == K).all()
    finally:
        pg.pgemm_destroy(h)
