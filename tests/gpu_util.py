"""Helpers for the GPU parity tests (host-side marshalling and comparison)."""
import numpy as np
import pytest

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def need_gpu():
    if torch is None or not torch.cuda.is_available():
        pytest.skip("no GPU available")
    from bit_mixed_precision_amd import bq

    bq.lib()  # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev):
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def f16_bits(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def ord16(bits: np.ndarray) -> np.ndarray:
    """Monotone integer image of fp16 bit patterns (+0 and -0 both map to 0)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def assert_f16_within_1ulp(got_bits: np.ndarray, want_bits: np.ndarray, what=""):
    """|ord16(got) - ord16(want)| <= 1 and no NaN; returns how many differ by 1.

    ord16 orders all fp16 values including the infinities, so an overflow to
    inf is one step from the largest finite value, and otherwise must match.
    """
    assert got_bits.shape == want_bits.shape
    g_nan = ((got_bits & 0x7C00) == 0x7C00) & ((got_bits & 0x3FF) != 0)
    assert not g_nan.any(), f"{what}: NaN in GPU output"
    d = np.abs(ord16(got_bits) - ord16(want_bits))
    bad = d > 1
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs off by more than 1 ulp; "
                           f"first at {np.argwhere(bad)[0]}: got {got_bits[bad][0]:#06x} "
                           f"want {want_bits[bad][0]:#06x}")
    return int((d == 1).sum())


def banner(msg: str):
    print(f"\n[gpu case] {msg}", flush=True)
