"""GPU: the allocation-free entry point pgemm_run_noalloc against pgemm_run.

pgemm_run_noalloc keeps stream-K partial tiles in a fixed device array
instead of a workspace the handle allocates. Through the C ABI, on the same
operands, its C must equal pgemm_run's bitwise (and the oracle's, bit-exact,
on small-integer inputs), every tile must be written once, on two calls in a
row with the second smaller than the first; splits that need more than the
array are refused before any launch, and the other modes, which need no
scratch, give pgemm_run's bits too.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

SK = 4


@pytest.fixture(scope="module")
def pg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_macro_amd as pg
    return pg


def say(msg):
    print(msg, flush=True)


def run_pair(pg, h, M, N, K, dtype, mode, workload):
    dev = torch.device("cuda:0")
    dt = {"f16": 0, "bf16": 1}[dtype]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    A, B = si.operands(M, N, K, dtype, "small_int", workload=workload)
    want = oracle.round_to(oracle.gemm(si.bits(A), si.bits(B), dtype), dtype)
    Ad, Bd = A.to(dev), B.to(dev)
    info = pg.pgemm_query_launch(h, M, N, K, dt, mode, 0)
    outs = []
    for fn in (pg.pgemm_run, pg.pgemm_run_noalloc):
        C = torch.full((M, N), float("nan"), dtype=tdt, device=dev)
        vis = torch.zeros(info["tiles"], dtype=torch.int32, device=dev)
        pg.pgemm_set_tile_counter(h, vis)
        try:
            fn(h, Ad, Bd, C, M, N, K, dt, mode, 0)
            torch.cuda.synchronize()
        finally:
            pg.pgemm_set_tile_counter(h, None)
        assert bool(torch.all(vis == 1)), (fn.__name__, M, N, K, mode)
        outs.append(si.bits(C.cpu()))
    assert np.array_equal(outs[0], outs[1]), (M, N, K, mode)
    assert np.array_equal(outs[1], want), (M, N, K, mode)


def test_noalloc_matches_run_on_two_calls_second_smaller(pg):
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(h, pg.PGEMM_TILE_128)
        # first call: 2176^2 x 1024 at 128^2 tiles, one whole wave plus 33 split tail tiles (~50 MiB of
        # partial tiles); second, smaller: 512^2 x 2048, sixteen tiles each split over workgroups
        for (M, N, K, dtype, wl) in [(2176, 2176, 1024, "f16", 41), (512, 512, 2048, "bf16", 42)]:
            split = pg.pgemm_query_streamk(h, M, N, K, {"f16": 0, "bf16": 1}[dtype], 0)
            say(f"case noalloc stream-K {M}x{N}x{K} {dtype}: {split}")
            assert split["pieces_split"] > 0
            assert 0 < split["workspace_bytes"] <= pg.PGEMM_NOALLOC_SCRATCH_BYTES
            run_pair(pg, h, M, N, K, dtype, SK, wl)
        # the modes that need no scratch
        for mode in (0, 1, 2, 3):
            say(f"case noalloc mode {mode}")
            run_pair(pg, h, 1000, 1032, 520, "f16", mode, 43)
    finally:
        pg.pgemm_destroy(h)


def test_noalloc_refuses_splits_beyond_its_scratch(pg):
    """A split needing more partial-tile bytes than the scratch holds fails before any launch
    (C untouched); pgemm_run, which may allocate, still runs it."""
    h = pg.pgemm_create(0)
    try:
        pg.pgemm_set_tile_config(h, pg.PGEMM_TILE_256)
        M = N = 6144
        K = 8192  # 576 tiles of 256^2 on 768 workgroups (grid multiple 3): every tile split, 336 MiB
        need = pg.pgemm_query_streamk(h, M, N, K, 0, 3)["workspace_bytes"]
        say(f"case noalloc refuse: needs {need} bytes")
        assert need > pg.PGEMM_NOALLOC_SCRATCH_BYTES
        dev = torch.device("cuda:0")
        A = torch.zeros((M, K), dtype=torch.float16, device=dev)
        B = torch.zeros((K, N), dtype=torch.float16, device=dev)
        C = torch.full((M, N), 3.0, dtype=torch.float16, device=dev)
        with pytest.raises(pg.PgemmError) as e:
            pg.pgemm_run_noalloc(h, A, B, C, M, N, K, 0, SK, 3)
        assert e.value.status == pg.PGEMM_ERR_UNSUPPORTED
        assert "scratch" in str(e.value)
        torch.cuda.synchronize()
        assert bool(torch.all(C == 3.0))
    finally:
        pg.pgemm_destroy(h)
