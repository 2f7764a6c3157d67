"""Work and traffic model for the quantized-GEMM path, and MI355X peaks.

The model follows the page "JAX Pallas 在 TPU 上编写高效矩阵乘法内核" (JAX Pallas
matmul kernels on TPU), section "矩阵乘法性能分析 / FLOPs 与内存带宽": a matmul
costs 2*m*k*n operations, and its minimum memory traffic is every input read
once plus the output written once.  With mixed operand widths each operand is
counted at its own width (B at bits/8 bytes per element, fp16 scale and
output at 2 bytes, int32 output at 4).  These are ALGORITHMIC quantities: the
re-reads a tiled kernel makes are not counted here (they show up in the
hardware counters instead).
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
HBM_PEAK_BYTES_PER_S = 8.0e12
INT8_MFMA_PEAK_OPS_PER_S = 5.0e15
FP16_MFMA_PEAK_FLOPS = 2.5e15
FP32_VECTOR_PEAK_FLOPS = 157.3e12


def gemm_ops(M: int, N: int, K: int) -> int:
    """Multiply-adds counted twice: 2 M N K."""
    return 2 * M * N * K


def operand_bytes(M: int, N: int, K: int, a_bytes: float, b_bits: int, out_bytes: int,
                  scale_bytes: int = 0) -> int:
    """Every operand moved once at its own width: A [M, K] at a_bytes per
    element, B [N, K] at b_bits, a per-column scale [N] at scale_bytes, the
    output [M, N] at out_bytes."""
    return int(M * K * a_bytes) + (N * K * b_bits) // 8 + N * scale_bytes + M * N * out_bytes


def gemm_bytes(M: int, N: int, K: int, bits: int, out: str = "f16") -> int:
    """A int8 [M,K] + B at `bits` [N,K] + fp16 scale [N] (f16 output only)
    + output [M,N] (fp16 or int32)."""
    if out == "f16":
        return operand_bytes(M, N, K, 1, bits, 2, scale_bytes=2)
    return operand_bytes(M, N, K, 1, bits, 4)


def nf4_gemm_bytes(M: int, N: int, K: int, zero: bool = True) -> int:
    """W4A16: fp16 A [M,K] + 4-bit codes [N,K] + fp16 scale (and zero point)
    [N] + fp16 output [M,N]."""
    return 2 * M * K + (N * K) // 2 + (4 if zero else 2) * N + 2 * M * N


def quantize_bytes(rows: int, cols: int) -> int:
    """fp16 x read once, int8 codes and fp16 scales written once."""
    return rows * cols * 2 + rows * cols + rows * 2


def pack_bytes(n: int, k: int, bits: int) -> int:
    """int8 values read once, packed bytes written once."""
    return n * k + (n * k * bits) // 8


def bound(ops: float, nbytes: float):
    """Which roofline bounds a kernel with this work: ('hbm'|'mfma', seconds)."""
    t_mem = nbytes / HBM_PEAK_BYTES_PER_S
    t_ops = ops / INT8_MFMA_PEAK_OPS_PER_S
    return ("hbm", t_mem) if t_mem >= t_ops else ("mfma", t_ops)
