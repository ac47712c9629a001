"""Pins for the CPU oracle, independent of the oracle's own code.

Each pin compares the oracle with something fixed by the mathematics or by
an independent implementation: torch's and numpy's casts for the
decoders and encoders, exact rational arithmetic (``fractions``) on tiny
products, worked examples under tests/golden, numpy's int64 matmul for
small-integer inputs, and closed forms (zero, identity, permutation,
rank one). Shapes are non-square throughout so that a transposed operand
or a swapped index cannot pass.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- decoders: exhaustive against torch's casts --------------------------------------------

@pytest.mark.parametrize("dtype,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_decode_16bit_exhaustive(dtype, tdt):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(b, dtype)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(tdt).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros decode with their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_e4m3fn_exhaustive():
    b = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = oracle.decode(b, "e4m3fn")
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_e4m3fn_golden_table():
    for line in open(os.path.join(GOLDEN, "e4m3fn_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        h, v = line.split()
        got = oracle.decode(np.array([int(h, 16)], dtype=np.uint8), "e4m3fn")[0]
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v))


# ---- encoders: round to nearest even ---------------------------------------------------------

def _f16_neighbours():
    """Every finite positive fp16 value, and the midpoints between consecutive ones."""
    b = np.arange(0, 0x7C00, dtype=np.uint16)
    v = b.view(np.float16).astype(np.float64)
    mid = (v[:-1] + v[1:]) / 2.0  # exact in double
    return v, mid


def test_encode_f16_matches_numpy():
    v, mid = _f16_neighbours()
    rng = np.random.default_rng(0)
    rand = np.concatenate([rng.uniform(-70000, 70000, 20000),
                           rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 16, 20000)])
    for x in (v, -v, mid, -mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40), rand,
              np.array([65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0])):
        got = oracle.round_to(x, "f16")
        with np.errstate(over="ignore"):
            ref = x.astype(np.float16).view(np.uint16)
        assert np.array_equal(got, ref), x[got != ref][:5]


def test_encode_f16_ties_to_even():
    # 1 + 2^-11 is halfway between 1 and 1 + 2^-10: even mantissa (1.0) wins;
    # 1 + 3*2^-11 is halfway between 1+2^-10 and 1+2^-9: 1+2^-9 (even) wins.
    assert oracle.round_to(np.array([1 + 2.0 ** -11]), "f16")[0] == 0x3C00
    assert oracle.round_to(np.array([1 + 3 * 2.0 ** -11]), "f16")[0] == 0x3C02
    assert oracle.round_to(np.array([65520.0]), "f16")[0] == 0x7C00  # rounds up to inf
    assert oracle.round_to(np.array([2.0 ** -25]), "f16")[0] == 0x0000  # tie to even zero
    assert oracle.round_to(np.array([3 * 2.0 ** -25]), "f16")[0] == 0x0002


def test_encode_bf16_matches_torch():
    rng = np.random.default_rng(1)
    # float32-exact inputs, so torch's float32 -> bf16 cast is a single rounding
    f = np.concatenate([
        rng.standard_normal(50000).astype(np.float32) * np.float32(2.0) ** rng.integers(-100, 100, 50000).astype(np.float32),
        (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32),  # every finite bf16 >= 0
    ]).astype(np.float32)
    f = f[np.isfinite(f)]
    # add exact midpoints between consecutive bf16 values (9 significant bits: exact in fp32)
    b = np.arange(0, 0x7F7F, dtype=np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)
    for x in (f, -f, mids, -mids):
        got = oracle.round_to(x.astype(np.float64), "bf16")
        ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref), x[got != ref][:5]


# ---- the GEMM ----------------------------------------------------------------------------------

def _exact_gemm(Ad, Bd):
    M, K = Ad.shape
    N = Bd.shape[1]
    A = [[Fraction(float(x)) for x in row] for row in Ad]
    B = [[Fraction(float(x)) for x in row] for row in Bd]
    return [[sum((A[i][k] * B[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (5, 2, 31), (4, 6, 17)])
def test_gemm_exact_rational_uniform(dtype, shape):
    """U[-1,1] inputs and K < 32: entries are multiples of 2^-24 (fp16), 2^-23 (bf16, drawn
    on a 2^-23 grid) or 2^-9 (e4m3) with |x| <= 1, so every partial sum is a multiple of
    2^-48 / 2^-46 / 2^-18 below 32 in magnitude: at most 53 bits, exact in fp64."""
    M, N, K = shape
    A, B = si.operands(M, N, K, dtype, "uniform", workload=M * 100 + K)
    Ab, Bb = si.bits(A), si.bits(B)
    C = oracle.gemm(Ab, Bb, dtype)
    exact = _exact_gemm(oracle.decode(Ab, dtype), oracle.decode(Bb, dtype))
    assert C.shape == (M, N)
    for i in range(M):
        for j in range(N):
            assert Fraction(C[i, j]) == exact[i][j]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_full_range_within_fp64_bound(dtype):
    """Random finite bit patterns across the whole exponent range: the oracle's
    error against the exact sum stays within K * 2^-53 * sum|a||b| (fp64 summation bound)."""
    rng = np.random.default_rng(7)
    M, N, K = 4, 3, 9
    def finite(n):
        x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
        d = oracle.decode(x, dtype)
        return np.where(np.isfinite(d), x, np.uint16(0x3C00 if dtype == "f16" else 0x3F80))
    Ab = finite(M * K).reshape(M, K)
    Bb = finite(K * N).reshape(K, N)
    C = oracle.gemm(Ab, Bb, dtype)
    Ad, Bd = oracle.decode(Ab, dtype), oracle.decode(Bb, dtype)
    exact = _exact_gemm(Ad, Bd)
    absprod = np.abs(Ad) @ np.abs(Bd)
    for i in range(M):
        for j in range(N):
            if math.isinf(C[i, j]):
                continue  # bf16 products near 2^254 can overflow double's sum; not a rounding case
            err = abs(Fraction(C[i, j]) - exact[i][j])
            assert err <= Fraction(K) * Fraction(2) ** -53 * Fraction(float(absprod[i, j])) * 2


def _load_golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        key, *rest = line.split()
        vals[key] = [float(x) for x in rest]
    M, N, K = int(vals["M"][0]), int(vals["N"][0]), int(vals["K"][0])
    return (np.array(vals["A"]).reshape(M, K), np.array(vals["B"]).reshape(K, N),
            np.array(vals["C"]).reshape(M, N))


@pytest.mark.parametrize("name", ["gemm_small_integer.txt", "gemm_small_fraction.txt"])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
def test_gemm_golden(name, dtype):
    A, B, C = _load_golden(name)
    if dtype == "e4m3fn" and np.abs(B).max() > 8:
        B = B / 2  # keep every entry exact in e4m3 (3 fraction bits)
        C = C / 2
    tA = torch.from_numpy(A).to(torch.float32).to(si.TORCH_DTYPES[dtype])
    tB = torch.from_numpy(B).to(torch.float32).to(si.TORCH_DTYPES[dtype])
    assert np.array_equal(tA.double().numpy(), A) and np.array_equal(tB.double().numpy(), B)
    got = oracle.gemm(si.bits(tA), si.bits(tB), dtype)
    assert np.array_equal(got, C)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
def test_gemm_closed_forms(dtype):
    M, N, K = 6, 5, 7
    A, B = si.operands(M, N, K, dtype, "uniform", workload=3)
    Ab, Bb = si.bits(A), si.bits(B)
    Ad, Bd = oracle.decode(Ab, dtype), oracle.decode(Bb, dtype)
    tdt = si.TORCH_DTYPES[dtype]
    # zero
    Z = si.bits(torch.zeros(M, K).to(tdt))
    assert np.all(oracle.gemm(Z, Bb, dtype) == 0)
    # identity on the left (I_K * B = B) and on the right (A * I_K = A)
    IK = si.bits(torch.eye(K).to(tdt))
    assert np.array_equal(oracle.gemm(IK, Bb, dtype), Bd)
    assert np.array_equal(oracle.gemm(Ab, IK, dtype), Ad)
    # permutation on the left permutes rows of B
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    P = torch.zeros(K, K)
    P[np.arange(K), perm] = 1
    assert np.array_equal(oracle.gemm(si.bits(P.to(tdt)), Bb, dtype), Bd[perm])
    # rank one: A[i,k] = a_i, B[k,j] = b_j  =>  C[i,j] = K * a_i * b_j
    a = torch.tensor([0.0, 0.5, -0.5, 1.0, -1.0, 2.0])
    b = torch.tensor([-2.0, 1.0, 0.5, -1.0, 2.0])
    R1 = oracle.gemm(si.bits(a[:, None].expand(M, K).to(tdt)), si.bits(b[None, :].expand(K, N).to(tdt)), dtype)
    assert np.array_equal(R1, K * np.outer(a.numpy(), b.numpy()).astype(np.float64))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3fn"])
def test_gemm_small_integers_match_int64_matmul(dtype):
    M, N, K = 37, 29, 301
    A, B = si.operands(M, N, K, dtype, "small_int", workload=5)
    ref = A.to(torch.int64).numpy() @ B.to(torch.int64).numpy()
    got = oracle.gemm(si.bits(A), si.bits(B), dtype)
    assert np.array_equal(got, ref.astype(np.float64))


def test_gemm_scaled_e4m3_matches_exact_rational_dequantisation():
    """Per-tensor scales: each scaled code is scale * code, so C is the exact
    rational sum of (sA * a) * (sB * b); checked with fractions on small integers
    (exact in double), for power-of-two and general scales, rows included."""
    M, N, K = 7, 5, 19
    A, B = si.operands(M, N, K, "e4m3fn", "small_int", workload=9)
    a = A.to(torch.int64).numpy()
    b = B.to(torch.int64).numpy()
    for sa, sb in [(0.5, 4.0), (0.25, 0.125), (0.37, 1.9), (-3.0, 0.75)]:
        got = oracle.gemm(si.bits(A), si.bits(B), "e4m3fn", scale_a=sa, scale_b=sb)
        for i in range(M):
            for j in range(N):
                exact = sum(Fraction(sa) * int(a[i, k]) * Fraction(sb) * int(b[k, j]) for k in range(K))
                assert abs(Fraction(got[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50), (sa, sb, i, j)
        rows = [4, 0, 6]
        assert np.array_equal(oracle.gemm(si.bits(A), si.bits(B), "e4m3fn", rows=rows, scale_a=sa, scale_b=sb),
                              got[rows])


def test_gemm_rows_and_threads():
    M, N, K = 50, 33, 70
    A, B = si.operands(M, N, K, "f16", "uniform", workload=9)
    Ab, Bb = si.bits(A), si.bits(B)
    full1 = oracle.gemm(Ab, Bb, "f16", nthreads=1)
    full8 = oracle.gemm(Ab, Bb, "f16", nthreads=8)
    assert np.array_equal(full1, full8)
    rows = np.array([49, 0, 17, 17, 3])
    assert np.array_equal(oracle.gemm(Ab, Bb, "f16", rows=rows, nthreads=3), full1[rows])
    # against numpy's float64 matmul of the decoded operands (a library routine; may
    # sum in another order, so only close, not identical)
    ref = oracle.decode(Ab, "f16") @ oracle.decode(Bb, "f16")
    assert np.allclose(full1, ref, rtol=0, atol=1e-12)


def test_gemm_edge_sizes():
    A, B = si.operands(3, 4, 0, "bf16")
    assert np.array_equal(oracle.gemm(si.bits(A), si.bits(B), "bf16"), np.zeros((3, 4)))
    A, B = si.operands(0, 4, 5, "bf16")
    assert oracle.gemm(si.bits(A), si.bits(B), "bf16").shape == (0, 4)
    with pytest.raises(ValueError):
        oracle.gemm(si.bits(A), si.bits(B).T.copy(), "bf16")


# ---- the parity measure -------------------------------------------------------------------------

def test_normwise_error_known_values():
    ref = np.array([3.0, 4.0])
    c = oracle.round_to(np.array([3.0, 4.0]), "f16")
    assert oracle.normwise_error(c, "f16", ref) == 0.0
    c = oracle.round_to(np.array([3.0, 3.0]), "f16")
    assert oracle.normwise_error(c, "f16", ref) == pytest.approx(1.0 / 5.0, rel=0, abs=1e-15)
    z = np.zeros(3)
    assert oracle.normwise_error(oracle.round_to(np.array([0.0, -0.0, 0.0]), "bf16"), "bf16", z) == 0.0
    assert oracle.normwise_error(oracle.round_to(np.array([0.0, 1.0, 0.0]), "bf16"), "bf16", z) == math.inf


def test_tolerance_separates_rne_from_truncation():
    """bf16 output: rounding the exact product to nearest even sits near 1.7e-3,
    below the 2e-3 bound, while truncating fp32 to bf16 lands near 3.3e-3 and fails.
    The parity bound is therefore tight enough to catch a truncating epilogue."""
    M = N = 256
    K = 1024
    A, B = si.operands(M, N, K, "bf16", "uniform", workload=1)
    ref = oracle.gemm(si.bits(A), si.bits(B), "bf16")
    rne = oracle.round_to(ref, "bf16")
    e_rne = oracle.normwise_error(rne, "bf16", ref)
    trunc = (ref.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    e_trunc = oracle.normwise_error(trunc, "bf16", ref)
    assert 1.0e-3 < e_rne < 2.0e-3 < e_trunc


def test_small_integer_outputs_round_exactly():
    """Small-integer products are exact in fp32 and round once to the output type."""
    A, B = si.operands(20, 24, 511, "f16", "small_int", workload=4)
    ref = oracle.gemm(si.bits(A), si.bits(B), "f16")
    out = oracle.round_to(ref, "f16")
    assert np.array_equal(oracle.decode(out, "f16"), ref)  # |C| <= 4K = 2044: exact in fp16
