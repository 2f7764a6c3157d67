"""The fused epilogues' GELU (csrc/gelu_fit.h): the committed constants are
what csrc/gen_gelu_fit.py produces, and an fp32 emulation of the kernels'
GELU rounds to within one fp16 ulp of the exact GELU (scipy's erfc in double)
on a dense grid.  CPU only."""
import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_mixed_precision_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_gelu_fit", os.path.join(CSRC, "gen_gelu_fit.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _header():
    text = open(os.path.join(CSRC, "gelu_fit.h")).read()
    num = r"(-?[0-9.]+(?:e-?[0-9]+)?)f"
    consts = {k: np.float32(float(re.search(k + r" = " + num, text).group(1)))
              for k in ("kGeluVmax", "kGeluA", "kGeluE")}
    body = text[text.index("kGeluQ["):]
    return consts, np.array([float(v) for v in re.findall(num + ",", body)], np.float32)


def test_header_matches_generator():
    gen = _gen()
    consts, q = _header()
    assert np.array_equal(q, gen.fit())
    assert consts["kGeluVmax"] == gen.VMAX and consts["kGeluA"] == gen.A_T and consts["kGeluE"] == gen.E2


def test_fit_reduces_to_the_normal_cdf():
    """Q(1) = H(0) = erfc(0) / 2 = 1/2, and exp2(v^2 kGeluE) = exp(-v^2 / 2)."""
    gen = _gen()
    _, q = _header()
    assert abs(float(q.astype(np.float64).sum()) - 0.5) < 1e-4
    assert abs(2.0 ** (4.0 * float(gen.E2)) - np.exp(-2.0)) < 1e-7


def test_gelu_fp32_within_one_ulp():
    from scipy.special import erfc

    gen = _gen()
    _, q = _header()
    v = np.concatenate([np.linspace(-12, 12, 400001), [-6.0, -5.5, 0.0, 1e-3, -1e-3]]).astype(np.float32)
    got = gen.gelu_fp32(v, q).astype(np.float16).view(np.uint16).astype(np.int32)
    ref = (0.5 * v.astype(np.float64) * erfc(-v.astype(np.float64) / np.sqrt(2.0))).astype(np.float16)
    ref = ref.view(np.uint16).astype(np.int32)
    o = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    assert np.abs(o(got) - o(ref)).max() <= 1


def test_planted_error_is_caught():
    """The check fails for a fit one degree too low (errors of several fp16 ulps)."""
    from scipy.special import erfc

    gen = _gen()
    _, q = _header()
    v = np.linspace(-8, 8, 200001).astype(np.float32)
    bad = q.copy()
    bad[-1] = 0.0  # drop the highest-degree term
    got = gen.gelu_fp32(v, bad).astype(np.float16).view(np.uint16).astype(np.int32)
    ref = (0.5 * v.astype(np.float64) * erfc(-v.astype(np.float64) / np.sqrt(2.0))).astype(np.float16)
    ref = ref.view(np.uint16).astype(np.int32)
    o = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    assert np.abs(o(got) - o(ref)).max() > 1
