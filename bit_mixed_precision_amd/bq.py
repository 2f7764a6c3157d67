"""Thin ctypes binding of libbq.so (C ABI in include/bq.h).

Argument marshalling only: every function checks dtypes/devices/shapes of
torch tensors, allocates outputs when none are given, and calls the C entry
point of the same name on the current torch stream of the tensors' device.
All compute runs in the HIP kernels of libbq.so; there is no fallback: if the
library is missing or the device is not gfx950 the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbq.so")

BQ_OK, BQ_ERR_NULL, BQ_ERR_SHAPE, BQ_ERR_ALIGN, BQ_ERR_HIP, BQ_ERR_DEVICE, BQ_ERR_ARG = range(7)
PATH_AUTO, PATH_STREAM, PATH_TILED, PATH_GEMV = 0, 1, 2, 3
MAX_K = 65536
_PATHS = {"auto": PATH_AUTO, "stream": PATH_STREAM, "tiled": PATH_TILED, "gemv": PATH_GEMV}

# (name, argtypes) for every entry point declared in include/bq.h
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "bq_version": [],
    "bq_status_string": [_I],
    "bq_quantize_rows": [_P, _I64, _I64, _P, _P, _P],
    "bq_pack_int4": [_P, _I64, _I64, _P, _P],
    "bq_pack_int2": [_P, _I64, _I64, _P, _P],
    "bq_gemm_w8a8_dequant": [_P, _P, _P, _P, _I64, _I64, _I64, _P],
    "bq_gemm_w4a8_dequant": [_P, _P, _P, _P, _I64, _I64, _I64, _P],
    "bq_gemm_w2a8_dequant": [_P, _P, _P, _P, _I64, _I64, _I64, _P],
    "bq_gemm_w8a8_i32": [_P, _P, _P, _I64, _I64, _I64, _P],
    "bq_gemm_w4a8_i32": [_P, _P, _P, _I64, _I64, _I64, _P],
    "bq_gemm_w2a8_i32": [_P, _P, _P, _I64, _I64, _I64, _P],
    "bq_gemm": [_P, _P, _I, _P, _P, _I64, _I64, _I64, _I, _P],
    "bq_gemm_dual_scale": [_P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I, _P],
    "bq_gemm_batched": [_P, _I64, _P, _I64, _I, _P, _I64, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P],
    "bq_gemm_act": [_P, _P, _I, _P, _P, _I, _P, _I64, _I64, _I64, _I, _P],
    "bq_quantize_rows_bits": [_P, _I64, _I64, _I, _P, _P, _P],
    "bq_quantize_pack": [_P, _I64, _I64, _I, _P, _P, _P],
    "bq_gemm_select_path": [_I64, _I64, _I64, _I],
    "bq_gemm_nf4_a16": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P],
    "bq_gemm_splitk_workspace_bytes": [_I64, _I64, _I64, _I],
    "bq_gemm_splitk": [_P, _P, _I, _P, _P, _I64, _I64, _I64, _P, _I64, _P],
    "bq_gemm_splitk_static": [_P, _P, _I, _P, _P, _I64, _I64, _I64, _P],
}
_RESTYPES = {"bq_status_string": ctypes.c_char_p, "bq_gemm_splitk_workspace_bytes": ctypes.c_int64}


class BQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libbq.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, ctypes.c_int)
        _lib = handle
    return _lib


def version() -> int:
    return lib().bq_version()


def status_string(status: int) -> str:
    return lib().bq_status_string(status).decode()


def select_path(M: int, N: int, K: int, bits: int) -> str:
    p = lib().bq_gemm_select_path(M, N, K, bits)
    return {PATH_STREAM: "stream", PATH_TILED: "tiled", PATH_GEMV: "gemv"}[p]


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _check_tensor(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(name: str, device: torch.device, *args):
    with torch.cuda.device(device):
        st = getattr(lib(), name)(*args, _stream(device))
    if st != BQ_OK:
        raise BQError(st, name)


# --------------------------------------------------------------------------
# public functions (same names as the C entry points, without the prefix)
# --------------------------------------------------------------------------

def quantize_rows(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                  scale: Optional[torch.Tensor] = None):
    """Per-row int8 quantization of fp16 x [rows, cols] -> (q int8, scale fp16 [rows])."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    _check_tensor(x, "x", torch.float16)
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float16, device=dev)
    _check_tensor(q, "q", torch.int8, (rows, cols), dev)
    _check_tensor(scale, "scale", torch.float16, (rows,), dev)
    _call("bq_quantize_rows", dev, _ptr(x), rows, cols, _ptr(q), _ptr(scale))
    return q, scale


def quantize_rows_bits(x: torch.Tensor, bits: int, q: Optional[torch.Tensor] = None,
                       scale: Optional[torch.Tensor] = None):
    """Per-row quantization of fp16 x [rows, cols] to the code range of a
    weight format, qmax = 2^(bits-1) - 1 (bits 8, 4, 2) -> (q int8, scale fp16
    [rows]); the codes feed pack_int4 / pack_int2."""
    if bits not in (8, 4, 2):
        raise ValueError("bits must be 8, 4 or 2")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    _check_tensor(x, "x", torch.float16)
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float16, device=dev)
    _check_tensor(q, "q", torch.int8, (rows, cols), dev)
    _check_tensor(scale, "scale", torch.float16, (rows,), dev)
    _call("bq_quantize_rows_bits", dev, _ptr(x), rows, cols, bits, _ptr(q), _ptr(scale))
    return q, scale


def quantize_pack(x: torch.Tensor, bits: int, out: Optional[torch.Tensor] = None,
                  scale: Optional[torch.Tensor] = None):
    """Per-row quantization of fp16 x [rows, cols] to the int4 (bits 4) or
    ternary (bits 2) code range, written packed -> (packed uint8 [rows,
    cols*bits/8], scale fp16 [rows]); equal to quantize_rows_bits followed by
    pack_int4 / pack_int2, in one pass."""
    if bits not in (4, 2):
        raise ValueError("bits must be 4 or 2")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    if cols % (8 // bits):
        raise ValueError(f"cols must be a multiple of {8 // bits}")
    _check_tensor(x, "x", torch.float16)
    dev = x.device
    if out is None:
        out = torch.empty((rows, cols * bits // 8), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float16, device=dev)
    _check_tensor(out, "out", torch.uint8, (rows, cols * bits // 8), dev)
    _check_tensor(scale, "scale", torch.float16, (rows,), dev)
    _call("bq_quantize_pack", dev, _ptr(x), rows, cols, bits, _ptr(out), _ptr(scale))
    return out, scale


def _pack(name: str, factor: int, v: torch.Tensor, out: Optional[torch.Tensor]):
    if v.dim() != 2:
        raise ValueError("v must be 2-D [n, k]")
    n, k = v.shape
    _check_tensor(v, "v", torch.int8)
    if k % factor:
        raise ValueError(f"k must be a multiple of {factor}")
    if out is None:
        out = torch.empty((n, k // factor), dtype=torch.uint8, device=v.device)
    _check_tensor(out, "out", torch.uint8, (n, k // factor), v.device)
    _call(name, v.device, _ptr(v), n, k, _ptr(out))
    return out


def pack_int4(v: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 values in [-8, 7] [n, k] -> uint8 [n, k/2] (low nibble = even k)."""
    return _pack("bq_pack_int4", 2, v, out)


def pack_int2(v: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 values in [-2, 1] [n, k] -> uint8 [n, k/4] (code v+2, bits 2j = k%4 j)."""
    return _pack("bq_pack_int2", 4, v, out)


def _gemm_args(A, B, bits, scale, out):
    if bits not in (8, 4, 2):
        raise ValueError("bits must be 8, 4 or 2")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N = B.shape[0]
    dev = A.device
    _check_tensor(A, "A", torch.int8)
    _check_tensor(B, "B", torch.int8 if bits == 8 else torch.uint8, (N, K * bits // 8), dev)
    if scale is not None:
        _check_tensor(scale, "scale", torch.float16, (N,), dev)
    odt = torch.float16 if scale is not None else torch.int32
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=dev)
    _check_tensor(out, "out", odt, (M, N), dev)
    return M, N, K, dev, out


def gemm(A: torch.Tensor, B: torch.Tensor, bits: int, scale: Optional[torch.Tensor] = None,
         out: Optional[torch.Tensor] = None, path: str = "auto") -> torch.Tensor:
    """C = A . B^T (int32), or fp16(C * scale[n]) when scale is given, with an
    explicit kernel path ("auto", "gemv", "stream" or "tiled").

    A int8 [M, K]; B int8 [N, K] (bits=8) or uint8 [N, K*bits/8] (bits=4, 2).
    """
    M, N, K, dev, out = _gemm_args(A, B, bits, scale, out)
    _call("bq_gemm", dev, _ptr(A), _ptr(B), bits, _ptr(scale), _ptr(out), M, N, K, _PATHS[path])
    return out


def gemm_splitk_workspace_bytes(M: int, N: int, K: int, bits: int) -> int:
    """Device workspace bytes gemm_splitk uses to split K for this shape (0:
    it would not split)."""
    n = lib().bq_gemm_splitk_workspace_bytes(M, N, K, bits)
    if n < 0:
        raise BQError(-n, "bq_gemm_splitk_workspace_bytes")
    return n


def gemm_splitk(A: torch.Tensor, B: torch.Tensor, bits: int, scale: Optional[torch.Tensor],
                workspace: Optional[torch.Tensor], out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gemm on the tiled path with K split over workgroups when the output
    has few tiles, using the caller's workspace (a uint8 device tensor whose
    first 4096 bytes are zero before the first call, e.g. torch.zeros of
    gemm_splitk_workspace_bytes(M, N, K, bits) bytes; None: no split)."""
    M, N, K, dev, out = _gemm_args(A, B, bits, scale, out)
    nbytes = 0
    if workspace is not None:
        _check_tensor(workspace, "workspace", torch.uint8, None, dev)
        nbytes = workspace.numel()
    _call("bq_gemm_splitk", dev, _ptr(A), _ptr(B), bits, _ptr(scale), _ptr(out), M, N, K, _ptr(workspace),
          nbytes)
    return out


def gemm_splitk_static(A: torch.Tensor, B: torch.Tensor, bits: int, scale: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gemm_splitk with the library's own static scratch (no device memory
    is allocated by the call; pass `out` as well to allocate nothing here).
    Calls that may overlap on one GPU race: order them on one stream."""
    M, N, K, dev, out = _gemm_args(A, B, bits, scale, out)
    _call("bq_gemm_splitk_static", dev, _ptr(A), _ptr(B), bits, _ptr(scale), _ptr(out), M, N, K)
    return out


def gemm_dual_scale(A: torch.Tensor, B: torch.Tensor, bits: int, w_scale: torch.Tensor,
                    x_scale: torch.Tensor, out: Optional[torch.Tensor] = None,
                    path: str = "auto") -> torch.Tensor:
    """fp16(acc[m,n] * w_scale[n] * x_scale[m]): the GEMM of a linear layer
    whose M activation rows were quantized per token (codes A, scales x_scale
    from quantize_rows)."""
    M, N, K, dev, out = _gemm_args(A, B, bits, w_scale, out)
    _check_tensor(x_scale, "x_scale", torch.float16, (M,), dev)
    _call("bq_gemm_dual_scale", dev, _ptr(A), _ptr(B), bits, _ptr(w_scale), _ptr(x_scale),
          _ptr(out), M, N, K, _PATHS[path])
    return out


ACTS = {"none": 0, "relu": 1, "gelu": 2}


def gemm_act(A: torch.Tensor, B: torch.Tensor, bits: int, w_scale: torch.Tensor,
             x_scale: Optional[torch.Tensor] = None, act: str = "gelu",
             out: Optional[torch.Tensor] = None, path: str = "auto") -> torch.Tensor:
    """fp16(act(acc[m,n] * w_scale[n] * x_scale[m])) with act "none", "relu"
    or "gelu" fused into the epilogue (x_scale None = 1)."""
    if act not in ACTS:
        raise ValueError(f"act must be one of {sorted(ACTS)}")
    M, N, K, dev, out = _gemm_args(A, B, bits, w_scale, out)
    if x_scale is not None:
        _check_tensor(x_scale, "x_scale", torch.float16, (M,), dev)
    _call("bq_gemm_act", dev, _ptr(A), _ptr(B), bits, _ptr(w_scale), _ptr(x_scale), ACTS[act],
          _ptr(out), M, N, K, _PATHS[path])
    return out


def linear(x: torch.Tensor, B: torch.Tensor, bits: int, w_scale: torch.Tensor,
           act: str = "none", path: str = "auto") -> torch.Tensor:
    """fp16 activations x [M, K] through a quantized weight: per-token int8
    quantization of x (quantize_rows), then the two-scale GEMM with the
    activation act fused."""
    q, xs = quantize_rows(x)
    if act == "none":
        return gemm_dual_scale(q, B, bits, w_scale, xs, path=path)
    return gemm_act(q, B, bits, w_scale, xs, act=act, path=path)


def gemm_batched(A: torch.Tensor, B: torch.Tensor, bits: int, scale: Optional[torch.Tensor] = None,
                 x_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 path: str = "auto") -> torch.Tensor:
    """Batched GEMM in one launch: B [batch, N, K*bits/8]; A [M, K] shared by
    every batch (broadcast, the fused-QKV shape) or [batch, M, K]; scale
    [batch, N] for the fp16 output (times x_scale [M], shared, when given),
    else int32.  Returns [batch, M, N]."""
    if bits not in (8, 4, 2):
        raise ValueError("bits must be 8, 4 or 2")
    if B.dim() != 3 or A.dim() not in (2, 3):
        raise ValueError("B must be [batch, N, K*bits/8] and A [M, K] or [batch, M, K]")
    batch, N, Kb = B.shape
    M, K = A.shape[-2:]
    dev = A.device
    _check_tensor(A, "A", torch.int8, (M, K) if A.dim() == 2 else (batch, M, K), dev)
    _check_tensor(B, "B", torch.int8 if bits == 8 else torch.uint8, (batch, N, K * bits // 8), dev)
    if scale is not None:
        _check_tensor(scale, "scale", torch.float16, (batch, N), dev)
    if x_scale is not None:
        if scale is None:
            raise ValueError("x_scale needs scale")
        _check_tensor(x_scale, "x_scale", torch.float16, (M,), dev)
    odt = torch.float16 if scale is not None else torch.int32
    if out is None:
        out = torch.empty((batch, M, N), dtype=odt, device=dev)
    _check_tensor(out, "out", odt, (batch, M, N), dev)
    strideA = 0 if A.dim() == 2 else M * K
    _call("bq_gemm_batched", dev, _ptr(A), strideA, _ptr(B), N * Kb, bits, _ptr(scale),
          N if scale is not None else 0, _ptr(x_scale), _ptr(out), M * N, batch, M, N, K, _PATHS[path])
    return out


def _named_dequant(bits, A, B, scale, out):
    if scale is None:
        raise ValueError("scale is required")
    M, N, K, dev, out = _gemm_args(A, B, bits, scale, out)
    _call(f"bq_gemm_w{bits}a8_dequant", dev, _ptr(A), _ptr(B), _ptr(scale), _ptr(out), M, N, K)
    return out


def _named_i32(bits, A, B, out):
    M, N, K, dev, out = _gemm_args(A, B, bits, None, out)
    _call(f"bq_gemm_w{bits}a8_i32", dev, _ptr(A), _ptr(B), _ptr(out), M, N, K)
    return out


def gemm_w8a8_dequant(A, B, scale, out=None):
    """fp16((A . B^T) * scale), B int8 [N, K]."""
    return _named_dequant(8, A, B, scale, out)


def gemm_w4a8_dequant(A, B, scale, out=None):
    """fp16((A . B^T) * scale), B packed int4 uint8 [N, K/2]."""
    return _named_dequant(4, A, B, scale, out)


def gemm_w2a8_dequant(A, B, scale, out=None):
    """fp16((A . B^T) * scale), B packed int2 uint8 [N, K/4]."""
    return _named_dequant(2, A, B, scale, out)


def gemm_w8a8_i32(A, B, out=None):
    return _named_i32(8, A, B, out)


def gemm_w4a8_i32(A, B, out=None):
    return _named_i32(4, A, B, out)


def gemm_w2a8_i32(A, B, out=None):
    return _named_i32(2, A, B, out)


def gemm_nf4_a16(A: torch.Tensor, B: torch.Tensor, scale: torch.Tensor,
                 zero: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W4A16 GEMM with NF4 weight codes: C = fp16(sum_k A[m,k] W[n,k]) with
    W[n,k] = fp16((nf4[code] - zero[n]) * scale[n]) and fp32 accumulation.

    A fp16 [M, K]; B uint8 [N, K/2] (code of k even in the low nibble);
    scale fp16 [N]; zero fp16 [N] or None (0)."""
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N = B.shape[0]
    dev = A.device
    _check_tensor(A, "A", torch.float16)
    _check_tensor(B, "B", torch.uint8, (N, K // 2), dev)
    _check_tensor(scale, "scale", torch.float16, (N,), dev)
    if zero is not None:
        _check_tensor(zero, "zero", torch.float16, (N,), dev)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    _check_tensor(out, "out", torch.float16, (M, N), dev)
    _call("bq_gemm_nf4_a16", dev, _ptr(A), _ptr(B), _ptr(scale), _ptr(zero), _ptr(out), M, N, K)
    return out
