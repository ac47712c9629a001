"""Seeded synthetic inputs shared by the tests, the smoke entry point and the bench.

This module only draws numbers and casts them to the storage formats; it
holds none of the GEMM's arithmetic. Both the GPU path and the CPU oracle
consume exactly the bit patterns returned here.

Recipe (persistent-matmul issue on the Triton tracker, "Describe the issue":
the sweeps are square M = N problems over a range of K):

* uniform[-1, 1]: a CPU ``torch.Generator`` seeded with ``seed`` draws
  ``rand(shape) * 2 - 1`` in float32, which is then cast with round to
  nearest even to the storage type (fp16, bf16, or OCP e4m3 with a
  per-tensor scale of 1.0, so dequantisation is the identity).
* normal(0, 1): the same generator draws ``randn`` in float32, then casts.
* small integers in {lo..hi}: ``randint`` then an exact cast; every
  partial sum of such a product is an integer, so it is exact in fp32.
* Seeds: operand A of workload c uses seed 2c, operand B seed 2c + 1.
* K sweeps draw A (M x Kmax) and B (Kmax x N) once and slice the leading
  K columns of A and the leading K rows of B.
"""
from __future__ import annotations

import numpy as np
import torch

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3fn": torch.float8_e4m3fn}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def uniform(shape, seed: int, dtype: str) -> torch.Tensor:
    x = torch.rand(tuple(shape), generator=_gen(seed), dtype=torch.float32) * 2.0 - 1.0
    return x.to(TORCH_DTYPES[dtype])


def normal(shape, seed: int, dtype: str) -> torch.Tensor:
    x = torch.randn(tuple(shape), generator=_gen(seed), dtype=torch.float32)
    return x.to(TORCH_DTYPES[dtype])


def small_int(shape, seed: int, dtype: str, lo: int = -2, hi: int = 2) -> torch.Tensor:
    x = torch.randint(lo, hi + 1, tuple(shape), generator=_gen(seed), dtype=torch.int32)
    return x.to(torch.float32).to(TORCH_DTYPES[dtype])


def draw(kind: str, shape, seed: int, dtype: str) -> torch.Tensor:
    if kind == "uniform":
        return uniform(shape, seed, dtype)
    if kind == "normal":
        return normal(shape, seed, dtype)
    if kind == "small_int":
        return small_int(shape, seed, dtype)
    raise ValueError(f"unknown input kind {kind!r}")


def operands(M: int, N: int, K: int, dtype: str, kind: str = "uniform", workload: int = 0):
    """(A, B) CPU tensors, A is M x K and B is K x N, seeds 2*workload and 2*workload + 1."""
    return (draw(kind, (M, K), 2 * workload, dtype), draw(kind, (K, N), 2 * workload + 1, dtype))


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU tensor as a numpy array (uint16 or uint8)."""
    t = t.contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    raise ValueError(f"unsupported element size {t.element_size()}")
