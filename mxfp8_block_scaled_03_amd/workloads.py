"""Seeded synthetic inputs for the MXFP8 workloads (shared by tests, smoke check and bench).

This module only draws random numbers: it holds none of the quantization or GEMM
arithmetic.  Every generator uses ``numpy.random.default_rng(seed)`` with the seed equal
to the workload number, draws in fp32 in the stated order, and rounds to bf16 (RNE,
torch's conversion) where the workload is bf16.  Weights are produced in the column-major
contract form ``[N][K]`` (a K x N matrix stored column by column) unless stated.

Workloads (transformer-shaped; the pages measure no public benchmark, so these stand in):
  1  M=256, K=512, N=256 fp32: X ~ N(0,1) except row 0 ~ U(-0.001, 0.001) and row 1
     with one +500 spike per 32-block; W ~ N(0, 0.02) in the pages' [K][N] form.
  2  projection M=8192, K=4096, N=4096 bf16: X ~ N(0,1) with 0.1% entries x100,
     W ~ N(0, 0.02).
  3  FFN pair, tokens 16384, hidden 5120, intermediate 8192 bf16: X ~ N(0,1),
     W1 [8192][5120], W2 [5120][8192] ~ N(0, 0.02), biases ~ N(0, 0.02) fp32.
  4  backward M=8192, K=4096, N=4096 bf16: X ~ N(0,1), W [N][K] ~ N(0, 0.02),
     dY = 1e-3 * Student-t(3).
  5  ragged/saturation M=4096, K=4000 (and companions), N=6144 bf16: X ~ Laplace(0,1)
     with 1% entries x1e4, W ~ N(0, 0.02).
  Q  standalone quantize of 2^28 bf16 = [16384][16384] ~ Laplace(0,1) with 1% x1e4.
"""
from __future__ import annotations

import numpy as np


def _bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def bf16_bits(t) -> np.ndarray:
    """uint16 bit patterns of a CPU bf16 tensor (the oracle's bf16 input form)."""
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def normal(rng, shape, std=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def with_outliers(rng, a: np.ndarray, frac: float, factor: float) -> np.ndarray:
    mask = rng.random(a.shape, dtype=np.float32) < frac
    a[mask] *= np.float32(factor)
    return a


def workload1(seed: int = 1):
    """X [256][512] fp32, W [512][256] fp32 (K x N, as in the pages' Y = XW)."""
    rng = np.random.default_rng(seed)
    M, K, N = 256, 512, 256
    x = normal(rng, (M, K))
    x[0] = rng.uniform(-0.001, 0.001, K).astype(np.float32)
    pos = rng.integers(0, 32, K // 32)
    x[1, 32 * np.arange(K // 32) + pos] = 500.0
    w_kn = normal(rng, (K, N), 0.02)
    return {"x": _f32(x), "w_kn": _f32(w_kn), "M": M, "K": K, "N": N}


def workload2(seed: int = 2, M: int = 8192, K: int = 4096, N: int = 4096):
    rng = np.random.default_rng(seed)
    x = with_outliers(rng, normal(rng, (M, K)), 0.001, 100.0)
    w = normal(rng, (N, K), 0.02)
    return {"x": _bf16(x), "w": _bf16(w), "M": M, "K": K, "N": N}


def workload3(seed: int = 3, T: int = 16384, H: int = 5120, I: int = 8192):
    rng = np.random.default_rng(seed)
    x = normal(rng, (T, H))
    w1 = normal(rng, (I, H), 0.02)
    w2 = normal(rng, (H, I), 0.02)
    b1 = normal(rng, (I,), 0.02)
    b2 = normal(rng, (H,), 0.02)
    return {"x": _bf16(x), "w1": _bf16(w1), "w2": _bf16(w2), "b1": _f32(b1), "b2": _f32(b2),
            "T": T, "H": H, "I": I}


def workload4(seed: int = 4, M: int = 8192, K: int = 4096, N: int = 4096):
    rng = np.random.default_rng(seed)
    x = normal(rng, (M, K))
    w = normal(rng, (N, K), 0.02)
    dy = (rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32)
    return {"x": _bf16(x), "w": _bf16(w), "dy": _bf16(dy), "M": M, "K": K, "N": N}


def workload5(seed: int = 5, M: int = 4096, K: int = 4000, N: int = 6144):
    rng = np.random.default_rng(seed)
    x = with_outliers(rng, rng.laplace(0.0, 1.0, (M, K)).astype(np.float32), 0.01, 1e4)
    w = normal(rng, (N, K), 0.02)
    return {"x": _bf16(x), "w": _bf16(w), "M": M, "K": K, "N": N}


def workload_q(seed: int = 6, rows: int = 16384, cols: int = 16384):
    rng = np.random.default_rng(seed)
    x = with_outliers(rng, rng.laplace(0.0, 1.0, (rows, cols)).astype(np.float32), 0.01, 1e4)
    return {"x": _bf16(x), "rows": rows, "cols": cols}
