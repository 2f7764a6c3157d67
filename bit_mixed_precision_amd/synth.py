"""Seeded synthetic inputs for the quantized-GEMM path.

This module only draws random numbers (numpy PCG64); it holds none of the
path's arithmetic (no quantization, packing, products or rounding to a
format other than the draw's own dtype cast) and imports nothing else from
this package, so both the HIP path and the oracle may consume what it makes.

Shapes and value distributions follow the workloads on the pages:
* BitBLAS custom-operator guide, section "测试与验证" (test): int8
  activations and int4-valued weights drawn uniformly, weights stored [N, K].
* BitBLAS guide, case 1: BitNet-b1.58 ternary weights {-1, 0, 1}.
* BMINF post-training quantization page, PartialAttention constructor: the
  fused QKV weight [3 * heads * dim_qkv, dim_in] quantized per output row.
Value ranges are inclusive ([-127, 127] for activations, [-8, 7] for int4).
"""
from __future__ import annotations

import numpy as np


def rng(seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def int8_uniform(g: np.random.Generator, shape, lo: int = -127, hi: int = 127) -> np.ndarray:
    return g.integers(lo, hi, shape, endpoint=True, dtype=np.int8)


def int4_values(g: np.random.Generator, shape) -> np.ndarray:
    """int8 array holding int4 values uniform in [-8, 7]."""
    return g.integers(-8, 7, shape, endpoint=True, dtype=np.int8)


def ternary_values(g: np.random.Generator, shape) -> np.ndarray:
    """int8 array of {-1, 0, 1} with probabilities {0.25, 0.5, 0.25}."""
    r = g.integers(0, 4, shape, dtype=np.int8)
    out = np.zeros(shape, np.int8)
    out[r == 0] = -1
    out[r == 3] = 1
    return out


def int2_values(g: np.random.Generator, shape) -> np.ndarray:
    """int8 array holding the full 2-bit code range [-2, 1]."""
    return g.integers(-2, 1, shape, endpoint=True, dtype=np.int8)


def fp16_uniform(g: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, n).astype(np.float16)


def fp16_normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float16)


# --------------------------------------------------------------------------
# Workload recipes (one generator per workload, draws in the listed order)
# --------------------------------------------------------------------------

def w4a8_case(M: int, N: int, K: int, seed: int = 0, scale_lo=0.001, scale_hi=0.01):
    """A int8 [M,K] in [-127,127]; B int4 values [N,K] in [-8,7]; fp16 scale [N]."""
    g = rng(seed)
    A = int8_uniform(g, (M, K))
    B = int4_values(g, (N, K))
    s = fp16_uniform(g, N, scale_lo, scale_hi)
    return A, B, s


def w2a8_case(M: int, N: int, K: int, seed: int = 0, scale_lo=0.5, scale_hi=2.0, ternary=True):
    """A int8 [M,K]; B ternary (or full 2-bit range) values [N,K]; fp16 scale [N]."""
    g = rng(seed)
    A = int8_uniform(g, (M, K))
    B = ternary_values(g, (N, K)) if ternary else int2_values(g, (N, K))
    s = fp16_uniform(g, N, scale_lo, scale_hi)
    return A, B, s


def w8a8_case(M: int, N: int, K: int, seed: int = 0, scale_lo=0.001, scale_hi=0.01):
    """A int8 [M,K]; B int8 [N,K] in [-127,127]; fp16 scale [N]."""
    g = rng(seed)
    A = int8_uniform(g, (M, K))
    B = int8_uniform(g, (N, K))
    s = fp16_uniform(g, N, scale_lo, scale_hi)
    return A, B, s


def bminf_weight(rows: int = 3 * 4096, cols: int = 4096, seed: int = 0, std: float = 0.02):
    """fp16 weight [rows, cols] ~ N(0, std): the fused QKV projection shape."""
    return fp16_normal(rng(seed), (rows, cols), std)


def bminf_linear_case(M: int = 64, rows: int = 3 * 4096, cols: int = 4096, seed: int = 0):
    """fp16 weight [rows, cols] ~ N(0, 0.02), then fp16 activations [M, cols]
    ~ N(0, 1) (the hidden state a linear layer quantizes per token)."""
    g = rng(seed)
    W = fp16_normal(g, (rows, cols), 0.02)
    X = fp16_normal(g, (M, cols), 1.0)
    return W, X


def bminf_case(M: int = 64, rows: int = 3 * 4096, cols: int = 4096, seed: int = 0):
    """fp16 weight [rows, cols] ~ N(0, 0.02), then int8 activations [M, cols]."""
    g = rng(seed)
    W = fp16_normal(g, (rows, cols), 0.02)
    A = int8_uniform(g, (M, cols))
    return W, A
