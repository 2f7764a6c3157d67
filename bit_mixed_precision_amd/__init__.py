"""MI355X (gfx950) quantized GEMM path: per-row int8 quantization, int4/int2
weight packing, and W8A8 / W4A8 / W2A8 integer GEMM with a fused fp16
per-output-channel scale.

The compute runs in the HIP library ``libbq.so`` (C ABI, declared in
``include/bq.h``); ``bit_mixed_precision_amd.bq`` is a thin ctypes binding
taking torch device tensors.  The binding is loaded on first use so that the
input generators (``synth``) and the work model (``roofline``) can be used
without a GPU.
"""
import importlib

__all__ = ["bq", "synth", "roofline"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
