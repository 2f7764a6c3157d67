"""The GELU epilogue's erfc fit (csrc/erfc_fit.h): the committed coefficients
are what csrc/gen_erfc_fit.py produces, and an fp32 emulation of the kernel's
GELU rounds to within one fp16 ulp of the exact GELU (scipy's erfc in double)
on a dense grid.  CPU only."""
import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_mixed_precision_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_erfc_fit", os.path.join(CSRC, "gen_erfc_fit.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _header_coeffs():
    text = open(os.path.join(CSRC, "erfc_fit.h")).read()
    body = text[text.index("kErfcFitC"):]
    return np.array([float(v) for v in re.findall(r"(-?[0-9.]+(?:e-?[0-9]+)?)f,", body)], np.float32)


def test_header_matches_generator():
    gen = _gen()
    assert np.array_equal(_header_coeffs(), gen.fit())


def test_gelu_fp32_within_one_ulp():
    from scipy.special import erfc

    gen = _gen()
    c = _header_coeffs()
    v = np.concatenate([np.linspace(-10, 10, 400001), [-6.0, -5.5, 0.0, 1e-3, -1e-3]]).astype(np.float32)
    got = gen.gelu_fp32(v, c).astype(np.float16).view(np.uint16).astype(np.int32)
    ref = (0.5 * v.astype(np.float64) * erfc(-v.astype(np.float64) / np.sqrt(2.0))).astype(np.float16)
    ref = ref.view(np.uint16).astype(np.int32)
    o = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    assert np.abs(o(got) - o(ref)).max() <= 1
