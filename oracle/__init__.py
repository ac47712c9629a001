"""CPU oracle for C = A*B (fp64, exact decoders) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke entry point and the benchmark's cpu_baseline
leg may import this package. The GPU product path never imports it, and it
imports nothing from the product path: it is built from `oracle.c` alone
with the host C compiler.

What it computes is the plain definition of the GEMM that a persistent
kernel tiles (persistent-kernel forum thread, question; KernelWiki
"Persistent Kernels with Cluster Launch Control", "Choosing between static
and CLC scheduling": scheduling adds no work and changes no value):

    C[i, j] = sum_k dec(A[i, k]) * dec(B[k, j])      in IEEE double, k ascending

with A (M x K), B (K x N), C (M x N) row-major and dec() the exact decoding
of IEEE binary16, bfloat16 or OCP E4M3 ("fn") bit patterns. Quantised e4m3
inputs with per-tensor scales sA, sB represent sA * dec(a) and sB * dec(b),
so their C is sA * sB times that sum.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f16": 0, "bf16": 1, "e4m3fn": 2}
_ITEMSIZE = {"f16": 2, "bf16": 2, "e4m3fn": 1}
OUT_DTYPES = {"f16": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O3", "-std=c99", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
             "-Wall", "-Wextra", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_e4m3fn.restype = ctypes.c_double
        lib.oracle_encode_f16_rne.argtypes = [ctypes.c_double]
        lib.oracle_encode_f16_rne.restype = ctypes.c_uint16
        lib.oracle_encode_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_encode_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_decode_array.argtypes = [vp, i64, ctypes.c_int, dp]
        lib.oracle_decode_array.restype = ctypes.c_int
        lib.oracle_round_array.argtypes = [dp, i64, ctypes.c_int, vp]
        lib.oracle_round_array.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, dp, ctypes.c_int]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm_rows.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, vp, i64, dp,
                                         ctypes.c_int]
        lib.oracle_gemm_rows.restype = ctypes.c_int
        lib.oracle_normwise_error.argtypes = [vp, ctypes.c_int, dp, i64]
        lib.oracle_normwise_error.restype = ctypes.c_double
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype not in DTYPES:
        raise ValueError(f"unknown input dtype {dtype!r}")
    want = np.uint8 if _ITEMSIZE[dtype] == 1 else np.uint16
    x = np.ascontiguousarray(x)
    if x.dtype.itemsize != _ITEMSIZE[dtype]:
        raise ValueError(f"{dtype} bit patterns need itemsize {_ITEMSIZE[dtype]}, got {x.dtype}")
    return x.view(want)


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact values of the stored bit patterns, as float64 (same shape)."""
    b = _bits(bits, dtype)
    out = np.empty(b.shape, dtype=np.float64)
    rc = _load().oracle_decode_array(b.ctypes.data, b.size, DTYPES[dtype], _dptr(out))
    if rc:
        raise RuntimeError(f"oracle_decode_array failed ({rc})")
    return out


def round_to(x: np.ndarray, out_dtype: str) -> np.ndarray:
    """Round float64 values to fp16/bf16, nearest-even; returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    rc = _load().oracle_round_array(_dptr(x), x.size, OUT_DTYPES[out_dtype], out.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_round_array failed ({rc})")
    return out


def gemm(A_bits: np.ndarray, B_bits: np.ndarray, dtype: str, rows=None, nthreads=None,
         scale_a: float = 1.0, scale_b: float = 1.0) -> np.ndarray:
    """fp64 C = dec(A) @ dec(B); with `rows`, only those rows of C (in that order).

    scale_a, scale_b: per-tensor scales of quantised inputs (the e4m3 workload's
    dequantisation, value = scale * decoded code). A scaled code times a scaled
    code is the two scales times the product of the codes, so the scaled sum is
    scale_a * scale_b times the unscaled one, applied here in double."""
    A = _bits(A_bits, dtype)
    B = _bits(B_bits, dtype)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} x {B.shape}")
    M, K = A.shape
    N = B.shape[1]
    nt = default_threads() if nthreads is None else int(nthreads)
    lib = _load()
    if rows is None:
        C = np.empty((M, N), dtype=np.float64)
        rc = lib.oracle_gemm(A.ctypes.data, B.ctypes.data, M, N, K, DTYPES[dtype], _dptr(C), nt)
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        C = np.empty((r.size, N), dtype=np.float64)
        rc = lib.oracle_gemm_rows(A.ctypes.data, B.ctypes.data, M, N, K, DTYPES[dtype],
                                  r.ctypes.data, r.size, _dptr(C), nt)
    if rc:
        raise RuntimeError(f"oracle gemm failed ({rc})")
    if scale_a != 1.0 or scale_b != 1.0:
        C *= float(scale_a) * float(scale_b)
    return C


def normwise_error(C_bits: np.ndarray, out_dtype: str, C_ref: np.ndarray) -> float:
    """||C - C_ref||_F / ||C_ref||_F with C given as fp16/bf16 bit patterns."""
    c = np.ascontiguousarray(C_bits).view(np.uint16)
    ref = np.ascontiguousarray(C_ref, dtype=np.float64)
    if c.size != ref.size:
        raise ValueError("size mismatch")
    return float(_load().oracle_normwise_error(c.ctypes.data, OUT_DTYPES[out_dtype], _dptr(ref),
                                               ref.size))
