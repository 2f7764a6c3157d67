"""Pins for the oracle's IEEE binary16 codec.

The codec is checked against numpy's own float16 conversions (an independent
library implementation of IEEE 754 binary16, correctly rounded) and against
exact rational arithmetic at every rounding midpoint.
"""
from fractions import Fraction

import numpy as np
import pytest


def test_decode_all_patterns(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros survive
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_encode_roundtrip_all_finite(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    back = oracle.f64_to_f16(vals[fin])
    assert np.array_equal(back, bits[fin])


def test_encode_midpoints_ties_to_even(oracle):
    """Every midpoint between adjacent positive finite fp16 values rounds to the
    neighbour with an even significand; nudged by one double ulp it rounds to
    the nearer neighbour.  Expected values come from Fractions, not numpy."""
    pos = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. 65504
    lo = pos[:-1].view(np.float16).astype(np.float64)
    hi = pos[1:].view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2  # exact in double
    assert all(Fraction(m) == (Fraction(a) + Fraction(b)) / 2
               for m, a, b in zip(mid[::997], lo[::997], hi[::997]))
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(oracle.f64_to_f16(mid), even)
    assert np.array_equal(oracle.f64_to_f16(np.nextafter(mid, 0)), pos[:-1])
    assert np.array_equal(oracle.f64_to_f16(np.nextafter(mid, np.inf)), pos[1:])
    # negative side mirrors the positive side
    assert np.array_equal(oracle.f64_to_f16(-mid), even | 0x8000)


def test_encode_overflow_and_underflow(oracle):
    cases = {
        65504.0: 0x7BFF,
        65519.99: 0x7BFF,
        65520.0: 0x7C00,  # midpoint to 2^16 rounds to even -> infinity
        1e30: 0x7C00,
        -65520.0: 0xFC00,
        2.0 ** -24: 0x0001,
        2.0 ** -25: 0x0000,  # tie between 0 and the smallest subnormal -> 0
        np.nextafter(2.0 ** -25, 1): 0x0001,
        3 * 2.0 ** -25: 0x0002,  # tie between 1 and 2 quanta -> 2
        2.0 ** -14 - 2.0 ** -25: 0x0400,  # tie between largest subnormal and 2^-14
        -0.0: 0x8000,
        float("inf"): 0x7C00,
        float("-inf"): 0xFC00,
    }
    for x, want in cases.items():
        assert int(oracle.f64_to_f16(np.array([x]))[0]) == want, x
    assert int(oracle.f64_to_f16(np.array([np.nan]))[0]) & 0x7FFF > 0x7C00


def test_encode_matches_numpy_on_float32_sample(oracle):
    """A strided sample of all float32 bit patterns (every 509th) plus random
    doubles, against numpy's correctly rounded conversion to float16."""
    pats = np.arange(0, 2**32, 509, dtype=np.uint64).astype(np.uint32)
    f = pats.view(np.float32)
    f = f[np.isfinite(f)]
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    got = oracle.f64_to_f16(f.astype(np.float64))
    assert np.array_equal(got, ref)
    g = np.random.default_rng(1)
    d = g.standard_normal(1_000_000) * np.exp(g.uniform(-25, 12, 1_000_000))
    with np.errstate(over="ignore"):
        ref = d.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f64_to_f16(d), ref)
