"""Pins for the oracle's per-row int8 quantization (BMINF post-training
quantization page, section 實現代碼分析2: scale = absmax / 127 stored as
fp16, codes = nearest integer of x / scale, symmetric).

Expected values are computed here with exact rational arithmetic (Fractions)
and Python's round-half-even, independently of the oracle's double code.
"""
from fractions import Fraction

import numpy as np
import pytest

from bit_mixed_precision_amd import synth


def _exact_f16(fr: Fraction) -> int:
    """Nearest fp16 (ties to even) of a non-negative rational, by brute force
    over the two fp16 neighbours bracketing it."""
    assert fr >= 0
    if fr >= 65520:
        return 0x7C00
    # candidate from a float approximation, then fix up with exact compares
    approx = int(np.array([float(fr)], np.float64).astype(np.float16).view(np.uint16)[0])
    best = None
    for c in range(max(0, approx - 2), min(0x7BFF, approx + 2) + 1):
        v = Fraction(float(np.uint16(c).view(np.float16)))
        d = abs(v - fr)
        key = (d, c % 2)  # nearer first, then even significand
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _exact_code(x: float, s: float) -> int:
    if s == 0:
        return 0
    q = round(Fraction(x) / Fraction(s))  # Fraction.__round__ rounds half to even
    return max(-127, min(127, q))


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def test_scale_exhaustive_over_all_absmax(oracle):
    """Every positive finite fp16 absmax: scale == RNE16(absmax/127) exactly."""
    a_bits = np.arange(1, 0x7C00, dtype=np.uint16)
    x = np.zeros((a_bits.size, 2), np.uint16)
    x[:, 0] = a_bits
    x[1::2, 0] |= 0x8000  # absmax of a negative value
    q, s = oracle.quantize_rows(x)
    a = _f16(a_bits)
    want = np.array([_exact_f16(Fraction(float(v)) / 127) for v in a], np.uint16)
    assert np.array_equal(s, want)


def test_codes_exact_on_random_rows(oracle):
    g = np.random.default_rng(7)
    x1 = synth.fp16_normal(g, (24, 97), 0.02)
    x2 = g.uniform(-3, 3, (24, 97)).astype(np.float16)
    x3 = (g.uniform(-1, 1, (8, 97)) * 2.0 ** -16).astype(np.float16)  # subnormal x
    x = np.concatenate([x1, x2, x3])
    q, s = oracle.quantize_rows(x)
    xs = x.astype(np.float64)
    ss = _f16(s)
    for r in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in xs[r])
        assert s[r] == _exact_f16(amax / 127)
        for k in range(x.shape[1]):
            assert q[r, k] == _exact_code(xs[r, k], ss[r]), (r, k)


def test_ties_round_to_even(oracle):
    s0 = 2.0 ** -7
    amax = 127 * s0  # representable, and amax/127 == s0 exactly
    halves = [0.5, 1.5, 2.5, 3.5, 125.5, 126.5, -0.5, -1.5, -2.5, -126.5]
    want = [0, 2, 2, 4, 126, 126, 0, -2, -2, -126]
    row = np.array([amax] + [h * s0 for h in halves], np.float16)
    assert np.array_equal(row.astype(np.float64)[1:], np.array(halves) * s0)
    q, s = oracle.quantize_rows(row[None, :])
    assert _f16(s)[0] == s0
    assert q[0, 0] == 127
    assert list(q[0, 1:]) == want


def test_invariants_on_bminf_shape(oracle):
    """max|q| == 127 on every row, |q*s - x| <= s/2 exactly, q in [-127,127]."""
    x = synth.bminf_weight(rows=1024, cols=4096, seed=0)
    q, s = oracle.quantize_rows(x)
    sd = _f16(s)
    assert np.all(sd >= 2.0 ** -14)  # normal scales at this distribution
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)
    err = np.abs(q.astype(np.float64) * sd[:, None] - x.astype(np.float64))
    assert np.all(err <= sd[:, None] / 2)  # products exact in double
    # the bound is reached (ties and exact halves do occur)
    assert np.isclose((err / (sd[:, None] / 2)).max(), 1.0)


def test_zero_tiny_and_subnormal_rows(oracle):
    q = 2.0 ** -24
    rows = np.array([
        [0.0, 0.0, -0.0, 0.0],
        [63 * q, -63 * q, q, 0.0],        # amax/127 < 2^-25 -> scale 0 -> codes 0
        [64 * q, -64 * q, 32 * q, q],     # scale = 2^-24 (subnormal)
        [189 * q, -189 * q, 100 * q, 0],  # scale 2^-24 too, |x/s| = 189 -> clamp
    ], np.float16)
    qq, s = oracle.quantize_rows(rows)
    assert list(s) == [0, 0, 1, 1]
    assert list(qq[0]) == [0, 0, 0, 0]
    assert list(qq[1]) == [0, 0, 0, 0]
    assert list(qq[2]) == [64, -64, 32, 1]
    assert list(qq[3]) == [127, -127, 100, 0]


def test_empty_and_nonfinite(oracle):
    q, s = oracle.quantize_rows(np.zeros((3, 0), np.float16))
    assert q.shape == (3, 0) and list(s) == [0, 0, 0]
    q, s = oracle.quantize_rows(np.zeros((0, 5), np.float16))
    assert q.shape == (0, 5) and s.shape == (0,)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_rows(np.array([[1.0, np.inf]], np.float16))
    with pytest.raises(oracle.OracleError):
        oracle.quantize_rows(np.array([[np.nan, 1.0]], np.float16))
