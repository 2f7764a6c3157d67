"""The oracle: plain CPU reference of the quantize -> pack -> integer GEMM ->
fp16 dequant path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  It shares no
code with the HIP library and never imports it.

Every function below is a thin numpy/ctypes wrapper around the plain C in
``bqref.c`` (argument checks and array allocation only); the arithmetic and
the order of its steps are those of the pages:

* "BMINF的後訓練量化實現" (BMINF post-training quantization), section
  實現代碼分析2 (PartialAttention.quantize and its quantize() docstring):
  per-row absmax / 127 fp16 scale, nearest-integer int8 codes, symmetric.
* "BitBLAS自定义操作开发指南：使用DSL扩展新的混合精度算子" (BitBLAS custom
  operator guide), sections 1 and 2 and cases 1 and 2: int8 x int4 / int2
  matmul with int32 accumulation over K of B stored [N, K], optional
  dequantization by a per-N fp16 scale, sub-byte weights stored as uint8
  [N, K/2].

Readings taken where the pages leave a step open are stated in the C source
and in the design notes: round-half-even of the exact quotient, codes clamped
to [-127, 127], zero scale -> zero codes, one correct rounding of acc*scale.

The submodule ``oracle.nf4`` (plain numpy) covers the W4A16 GEMM with NF4
weight codes, a per-row scale and zero point of the same BitBLAS guide
(case 2); its readings are stated in its own header.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_bqref.so")

OK, ERR_NULL, ERR_SHAPE, ERR_RANGE = 0, 1, 2, 3


class OracleError(RuntimeError):
    pass


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import _build

            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        for name, args in {
            "bqref_quantize_rows": [P, I64, I64, P, P],
            "bqref_quantize_rows_q": [P, I64, I64, ctypes.c_int, P, P],
            "bqref_pack_int4": [P, I64, I64, P],
            "bqref_unpack_int4": [P, I64, I64, P],
            "bqref_pack_int2": [P, I64, I64, P],
            "bqref_unpack_int2": [P, I64, I64, P],
            "bqref_gemm_i32": [P, P, P, I64, I64, I64],
            "bqref_dequant": [P, P, P, I64, I64],
            "bqref_dequant2": [P, P, P, P, I64, I64],
            "bqref_dequant_act": [P, P, P, ctypes.c_int, P, I64, I64],
        }.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.bqref_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.bqref_f16_to_f64.restype = ctypes.c_double
        lib.bqref_f64_to_f16.argtypes = [ctypes.c_double]
        lib.bqref_f64_to_f16.restype = ctypes.c_uint16
        lib.bqref_f16_to_f64_array.argtypes = [P, I64, P]
        lib.bqref_f16_to_f64_array.restype = None
        lib.bqref_f64_to_f16_array.argtypes = [P, I64, P]
        lib.bqref_f64_to_f16_array.restype = None
        lib.bqref_act.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.bqref_act.restype = ctypes.c_double
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(status: int, what: str):
    if status != OK:
        raise OracleError(f"{what}: oracle status {status}")


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _bits16(x) -> np.ndarray:
    """fp16 data as its uint16 bit patterns (accepts float16 or uint16)."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        return np.ascontiguousarray(x).view(np.uint16)
    return _c(x, np.uint16)


# --------------------------------------------------------------------------
# fp16 codec (IEEE 754 binary16)
# --------------------------------------------------------------------------

def f16_to_f64(h) -> np.ndarray:
    h = _bits16(h)
    out = np.empty(h.shape, np.float64)
    _load().bqref_f16_to_f64_array(_ptr(h), h.size, _ptr(out))
    return out


def f64_to_f16(d) -> np.ndarray:
    """Round doubles to the nearest fp16 (ties to even); returns uint16 bits."""
    d = np.ascontiguousarray(np.asarray(d, np.float64))
    out = np.empty(d.shape, np.uint16)
    _load().bqref_f64_to_f16_array(_ptr(d), d.size, _ptr(out))
    return out


# --------------------------------------------------------------------------
# steps of the path
# --------------------------------------------------------------------------

def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8 quantization of fp16 x [rows, cols].

    Returns (q int8 [rows, cols], scale as uint16 fp16 bits [rows]).
    BMINF page, section 實現代碼分析2, quantize(): scale = absmax/127 in fp16,
    q = nearest integer of x/scale.
    """
    x = _bits16(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows,), np.uint16)
    _check(_load().bqref_quantize_rows(_ptr(x), rows, cols, _ptr(q), _ptr(s)),
           "quantize_rows")
    return q, s


def quantize_rows_bits(x, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric quantization to the code range of `bits` (8, 4, 2):
    qmax = 2^(bits-1) - 1, scale = fp16(absmax/qmax), codes = nearest integer
    of x/scale clamped to [-qmax, qmax]; the BMINF page's int8 rule with the
    code range of the packed formats."""
    if bits not in (8, 4, 2):
        raise ValueError("bits must be 8, 4 or 2")
    x = _bits16(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows,), np.uint16)
    _check(_load().bqref_quantize_rows_q(_ptr(x), rows, cols, (1 << (bits - 1)) - 1, _ptr(q), _ptr(s)),
           "quantize_rows_bits")
    return q, s


def pack_int4(v) -> np.ndarray:
    """int8 values in [-8, 7], [N, K] -> uint8 [N, K/2]; low nibble = even k."""
    v = _c(v, np.int8)
    n, k = v.shape
    out = np.empty((n, k // 2), np.uint8)
    _check(_load().bqref_pack_int4(_ptr(v), n, k, _ptr(out)), "pack_int4")
    return out


def unpack_int4(p, k: int) -> np.ndarray:
    p = _c(p, np.uint8)
    n = p.shape[0]
    if p.shape != (n, k // 2):
        raise ValueError("packed shape does not match k")
    v = np.empty((n, k), np.int8)
    _check(_load().bqref_unpack_int4(_ptr(p), n, k, _ptr(v)), "unpack_int4")
    return v


def pack_int2(v) -> np.ndarray:
    """int8 values in [-2, 1], [N, K] -> uint8 [N, K/4]; code v+2, bits 2j = k%4 j."""
    v = _c(v, np.int8)
    n, k = v.shape
    out = np.empty((n, k // 4), np.uint8)
    _check(_load().bqref_pack_int2(_ptr(v), n, k, _ptr(out)), "pack_int2")
    return out


def unpack_int2(p, k: int) -> np.ndarray:
    p = _c(p, np.uint8)
    n = p.shape[0]
    if p.shape != (n, k // 4):
        raise ValueError("packed shape does not match k")
    v = np.empty((n, k), np.int8)
    _check(_load().bqref_unpack_int2(_ptr(p), n, k, _ptr(v)), "unpack_int2")
    return v


def gemm_i32(A, Bv) -> np.ndarray:
    """C[m,n] = sum_k A[m,k] * Bv[n,k] in int32 (BitBLAS page, section 1)."""
    A = _c(A, np.int8)
    Bv = _c(Bv, np.int8)
    M, K = A.shape
    N, K2 = Bv.shape
    if K != K2:
        raise ValueError("K mismatch")
    C = np.empty((M, N), np.int32)
    _check(_load().bqref_gemm_i32(_ptr(A), _ptr(Bv), _ptr(C), M, N, K), "gemm_i32")
    return C


def dequant(acc, scale) -> np.ndarray:
    """fp16(acc[m,n] * scale[n]) correctly rounded; returns uint16 bits."""
    acc = _c(acc, np.int32)
    scale = _bits16(scale)
    M, N = acc.shape
    if scale.shape != (N,):
        raise ValueError("scale must be [N]")
    out = np.empty((M, N), np.uint16)
    _check(_load().bqref_dequant(_ptr(acc), _ptr(scale), _ptr(out), M, N), "dequant")
    return out


def dequant2(acc, w_scale, x_scale) -> np.ndarray:
    """fp16(acc[m,n] * w_scale[n] * x_scale[m]) correctly rounded; uint16 bits.

    BMINF page, section 實現代碼分析2 (PartialAttention forward): per-token
    activation scale times per-channel weight scale times the int32 result."""
    acc = _c(acc, np.int32)
    w_scale = _bits16(w_scale)
    x_scale = _bits16(x_scale)
    M, N = acc.shape
    if w_scale.shape != (N,) or x_scale.shape != (M,):
        raise ValueError("w_scale must be [N] and x_scale [M]")
    out = np.empty((M, N), np.uint16)
    _check(_load().bqref_dequant2(_ptr(acc), _ptr(w_scale), _ptr(x_scale), _ptr(out), M, N),
           "dequant2")
    return out


ACTS = {"none": 0, "relu": 1, "gelu": 2}


def act(v: float, name: str) -> float:
    """The epilogue activation in double: identity, ReLU, or GELU
    v * Phi(v) with Phi(v) = erfc(-v / sqrt(2)) / 2."""
    return _load().bqref_act(float(v), ACTS[name])


def dequant_act(acc, w_scale, x_scale, name: str) -> np.ndarray:
    """fp16(act(acc[m,n] * w_scale[n] * x_scale[m])) rounded once (x_scale
    None = 1); uint16 bits.  JAX Pallas matmul page, fused-activation section:
    the activation on the wide result of the last K step, one downcast."""
    acc = _c(acc, np.int32)
    w_scale = _bits16(w_scale)
    M, N = acc.shape
    if w_scale.shape != (N,):
        raise ValueError("w_scale must be [N]")
    xp = None
    if x_scale is not None:
        x_scale = _bits16(x_scale)
        if x_scale.shape != (M,):
            raise ValueError("x_scale must be [M]")
        xp = _ptr(x_scale)
    out = np.empty((M, N), np.uint16)
    _check(_load().bqref_dequant_act(_ptr(acc), _ptr(w_scale), xp, ACTS[name], _ptr(out), M, N),
           "dequant_act")
    return out


def unpack(Bp, k: int, bits: int) -> np.ndarray:
    if bits == 8:
        return _c(Bp, np.int8)
    if bits == 4:
        return unpack_int4(Bp, k)
    if bits == 2:
        return unpack_int2(Bp, k)
    raise ValueError(bits)


def gemm_wxa8_i32(A, Bp, bits: int) -> np.ndarray:
    """Steps unpack -> integer GEMM for B stored as int8 [N,K] (bits=8) or
    packed uint8 [N, K*bits/8]."""
    K = np.asarray(A).shape[1]
    return gemm_i32(A, unpack(Bp, K, bits))


def gemm_wxa8_dequant(A, Bp, scale, bits: int) -> np.ndarray:
    """Steps unpack -> integer GEMM -> dequant; returns fp16 bits [M, N]."""
    return dequant(gemm_wxa8_i32(A, Bp, bits), scale)


def gemm_wxa8_dequant2(A, Bp, w_scale, x_scale, bits: int) -> np.ndarray:
    """Steps unpack -> integer GEMM -> two-scale dequant; fp16 bits [M, N]."""
    return dequant2(gemm_wxa8_i32(A, Bp, bits), w_scale, x_scale)


def gemm_batched(A, Bp, bits: int, scale=None, x_scale=None) -> np.ndarray:
    """Batched form of the path: for each batch z, unpack -> integer GEMM of
    A (shared [M, K], or A[z] of [batch, M, K]) with B[z] ([batch, N, K*bits/8])
    -> int32 [batch, M, N], or with scale [batch, N] the fp16 bits of the
    one-scale (or, with x_scale [M], two-scale) epilogue.

    BMINF page, section 實現代碼分析2: igemm of the fused QKV weight (3, N, K)
    with one activation (1, M, K) broadcast over the three weights."""
    A = np.asarray(A)
    Bp = np.asarray(Bp)
    batch = Bp.shape[0]
    out = []
    for z in range(batch):
        Az = A if A.ndim == 2 else A[z]
        acc = gemm_wxa8_i32(np.ascontiguousarray(Az), np.ascontiguousarray(Bp[z]), bits)
        if scale is None:
            out.append(acc)
        elif x_scale is None:
            out.append(dequant(acc, np.asarray(scale)[z]))
        else:
            out.append(dequant2(acc, np.asarray(scale)[z], x_scale))
    return np.stack(out)
