"""NF4 (4-bit NormalFloat) weights with fp16 activations: the oracle of the
W4A16 GEMM with a per-row scale and zero point.

TEST INFRASTRUCTURE ONLY (same rules as the rest of this package): only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; it shares no code with the HIP library.

Page: "BitBLAS自定义操作开发指南：使用DSL扩展新的混合精度算子" (BitBLAS custom
operator guide), case 2 (NF4 format): A fp16 [M, K]; B_nf4 uint8 [N, K/2]
(two 4-bit codes per byte along K); scale fp16 [N]; zero_point fp16 [N];
C[m, n] = sum_k float32(A[m, k]) * float32(B_dequantized[n, k]).  The page
leaves out both the NF4 table and the dequantization step.  Readings (stated
again in the design notes):

1. Codebook: the NF4 data type of the QLoRA paper (Dettmers et al., 2023,
   "4-bit NormalFloat"): quantiles of the standard normal distribution,
   eight on the positive side (probabilities evenly spaced from the offset
   down to one step above 1/2) and seven on the negative side (the same with
   seven steps), plus an exact zero, all divided by the largest, so the
   values run from -1 to 1.  The offset is the mean of 1 - 1/(2*15) and
   1 - 1/(2*16).  The sixteen values are held in fp16 (nearest), the type
   of the dequantized weights; code c selects the c-th smallest.
2. Codes: the low nibble of byte [n, k/2] is code k even, the high nibble
   k odd (the int4 layout of case 1), codes 0..15 unsigned.
3. Dequantization: W[n, k] = fp16(fp32(fp32(table[c] - zero[n]) * scale[n])),
   two fp32 operations in this order, one rounding to fp16 (nearest even);
   zero_point absent means 0.
4. Product: C[m, n] = fp16(sum_k A[m, k] * W[n, k]), the sum taken exactly
   and rounded once.  Every product of two fp16 values is exact in float64,
   and the float64 sum over K <= 65536 terms differs from the exact sum by at
   most K * 2^-53 * sum_k |A W|, far below the fp32 accumulation of a GPU;
   the tolerance used for GPU results (gemm_tolerance) is derived from the
   fp32 error bound.
"""
from __future__ import annotations

import numpy as np

NF4_OFFSET = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def nf4_codebook() -> np.ndarray:
    """The sixteen NF4 values in float64, ascending (reading 1)."""
    from scipy.special import ndtri

    pos = ndtri(np.linspace(NF4_OFFSET, 0.5, 9)[:-1])   # 8 quantiles above the median
    neg = -ndtri(np.linspace(NF4_OFFSET, 0.5, 8)[:-1])  # 7 below it
    v = np.sort(np.concatenate([pos, neg, [0.0]]))
    return v / v.max()


def nf4_table_f16() -> np.ndarray:
    """The codebook held in fp16: uint16 bit patterns, index = code."""
    return nf4_codebook().astype(np.float16).view(np.uint16)


def pack_codes(codes) -> np.ndarray:
    """uint8 codes [N, K] (0..15) -> bytes [N, K/2], low nibble = even k."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    if c.ndim != 2 or c.shape[1] % 2 or (c > 15).any():
        raise ValueError("codes must be [N, K] with K even and values 0..15")
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(p, k: int) -> np.ndarray:
    p = np.ascontiguousarray(p, dtype=np.uint8)
    out = np.empty((p.shape[0], k), np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def _f16(bits) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16)


def dequant_nf4(Bp, k: int, scale, zero=None) -> np.ndarray:
    """W [N, K] as fp16 bit patterns (reading 3)."""
    codes = unpack_codes(Bp, k)
    table = _f16(nf4_table_f16()).astype(np.float32)
    s = _f16(scale).astype(np.float32)[:, None]
    z = np.zeros_like(s) if zero is None else _f16(zero).astype(np.float32)[:, None]
    d = (table[codes] - z).astype(np.float32)   # one fp32 rounding
    w = (d * s).astype(np.float32)               # another
    return w.astype(np.float16).view(np.uint16)


def gemm_nf4_a16(A_f16, Bp, scale, zero=None):
    """C = fp16(sum_k A W) (reading 4).

    Returns (C as uint16 bits [M, N], the float64 sum S, and sum_k |A W|,
    both [M, N]) so that callers can apply gemm_tolerance."""
    A = _f16(A_f16).astype(np.float64)
    M, K = A.shape
    W = _f16(dequant_nf4(Bp, K, scale, zero)).astype(np.float64)
    S = A @ W.T
    absS = np.abs(A) @ np.abs(W).T
    C = S.astype(np.float16).view(np.uint16)
    return C, S, absS


def gemm_tolerance(S, absS, K: int) -> np.ndarray:
    """Largest |C_gpu - S| allowed for a GPU result C_gpu = fp16(S') where S'
    is any fp32 accumulation of the K exact products: |S' - S| <= gamma *
    sum|A W| with gamma = K u / (1 - K u), u = 2^-24 (each of at most K
    additions rounds once), plus the final rounding of S' to fp16, at most
    half an fp16 ulp of max(|S|, |S'|) -- bounded here by one ulp of
    |S| + gamma sum|A W| (subnormal spacing 2^-24 at the bottom)."""
    u = 2.0 ** -24
    gamma = K * u / (1.0 - K * u)
    acc_err = gamma * absS
    big = np.abs(S) + acc_err
    e = np.floor(np.log2(np.maximum(big, 2.0 ** -14)))
    ulp = 2.0 ** (e - 10)
    return acc_err + ulp
