"""Pins of the NF4 / W4A16 oracle (oracle/nf4.py) against things other than
itself: an independent construction of the codebook (bisection on CPython's
math.erfc instead of scipy's inverse normal), the quantile property checked
with the forward normal CDF, the published offset constant, exact rational
emulation of the fp32 dequantization steps, exhaustive packing, exact sums
(math.fsum of exact products), the blocked-K invariant, and the fp32
accumulation bound checked against a sequential fp32 sum."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4

# -- codebook ---------------------------------------------------------------


def _ppf_bisect(p: float) -> float:
    """Inverse of the standard normal CDF by bisection on Phi(x) =
    erfc(-x / sqrt 2) / 2 (CPython's libm), 200 halvings."""
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_offset_is_the_published_constant():
    # QLoRA (Dettmers et al., 2023): the NF4 construction uses the offset
    # 0.9677083, the mean of 1 - 1/30 and 1 - 1/32
    assert abs(nf4.NF4_OFFSET - 0.9677083) < 5e-8


def test_codebook_structure():
    v = nf4.nf4_codebook()
    assert v.shape == (16,)
    assert np.all(np.diff(v) > 0)
    assert v[0] == -1.0 and v[15] == 1.0 and v[7] == 0.0
    assert (v < 0).sum() == 7 and (v > 0).sum() == 8


def test_codebook_matches_independent_construction():
    off = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    step_p = (off - 0.5) / 8
    step_n = (off - 0.5) / 7
    pos = [_ppf_bisect(off - i * step_p) for i in range(8)]
    neg = [-_ppf_bisect(off - i * step_n) for i in range(7)]
    scale = max(pos)
    ref = sorted([x / scale for x in pos + neg] + [0.0])
    np.testing.assert_allclose(nf4.nf4_codebook(), ref, rtol=0, atol=1e-12)


def test_codebook_values_are_evenly_spaced_normal_quantiles():
    """Phi(c v) is evenly spaced in probability on each side (forward CDF,
    scipy.special.ndtr), with c the unnormalized largest value."""
    from scipy.special import ndtr

    v = nf4.nf4_codebook()
    c = _ppf_bisect(nf4.NF4_OFFSET)
    p_pos = ndtr(c * v[8:])          # 8 positive values, ascending
    p_neg = ndtr(-c * v[:7])         # 7 negative values, mirrored
    d_pos = np.diff(p_pos)
    d_neg = np.diff(p_neg)
    np.testing.assert_allclose(d_pos, (nf4.NF4_OFFSET - 0.5) / 8, rtol=0, atol=1e-12)
    np.testing.assert_allclose(d_neg, -(nf4.NF4_OFFSET - 0.5) / 7, rtol=0, atol=1e-12)
    assert abs(p_pos[0] - (0.5 + (nf4.NF4_OFFSET - 0.5) / 8)) < 1e-12
    assert abs(p_pos[-1] - nf4.NF4_OFFSET) < 1e-12


def test_table_f16():
    t = nf4.nf4_table_f16()
    assert t.dtype == np.uint16 and t.shape == (16,)
    assert t[0] == 0xBC00 and t[15] == 0x3C00 and t[7] == 0x0000
    # nearest fp16 of each value: no other fp16 is closer
    v = nf4.nf4_codebook()
    h = t.view(np.float16).astype(np.float64)
    for x, y in zip(v, h):
        up = np.nextafter(np.float16(y), np.float16(np.inf)).astype(np.float64)
        dn = np.nextafter(np.float16(y), np.float16(-np.inf)).astype(np.float64)
        assert abs(x - y) <= abs(x - up) and abs(x - y) <= abs(x - dn)


# -- packing ----------------------------------------------------------------


def test_pack_unpack_exhaustive():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = nf4.unpack_codes(b, 512)
    assert np.array_equal(codes[0, 0::2], np.arange(256) & 15)
    assert np.array_equal(codes[0, 1::2], np.arange(256) >> 4)
    assert np.array_equal(nf4.pack_codes(codes), b)
    # worked bytes: codes (1, 14) -> 0xE1, (15, 0) -> 0x0F
    assert nf4.pack_codes(np.array([[1, 14, 15, 0]], np.uint8)).tolist() == [[0xE1, 0x0F]]
    with pytest.raises(ValueError):
        nf4.pack_codes(np.array([[16, 0]], np.uint8))


# -- dequantization ---------------------------------------------------------


def _rne(x: Fraction, p: int, emin: int, maxv: Fraction):
    """x rounded to nearest (ties to even) in a binary format with p
    significand bits and minimum normal exponent emin; None = overflow."""
    if x == 0:
        return Fraction(0)
    s = 1 if x > 0 else -1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    q = a / Fraction(2) ** (e - (p - 1))
    n = math.floor(q)
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * Fraction(2) ** (e - (p - 1))
    if v > maxv:
        return None
    return s * v


F32MAX = Fraction((2 ** 24 - 1) * 2 ** 104)
F16MAX = Fraction(65504)


def _r32(x):
    return _rne(x, 24, -126, F32MAX)


def _r16(x):
    return _rne(x, 11, -14, F16MAX)


def _f16val(bits) -> Fraction:
    return Fraction(float(np.uint16(bits).view(np.float16)))


def _case(seed, N=7, K=64, wide=False):
    g = np.random.default_rng(seed)
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    if wide:  # scales and zero points over the whole fp16 range, subnormals included
        s = np.float16(g.choice([1, -1], N)) * np.float16(2.0) ** g.integers(-24, 15, N).astype(np.float16)
        z = np.float16(g.choice([1, -1], N)) * np.float16(2.0) ** g.integers(-24, 10, N).astype(np.float16)
        s = (s * np.float16(1 + g.integers(0, 1024, N) / 1024)).astype(np.float16)
    else:
        s = g.uniform(0.001, 0.01, N).astype(np.float16)
        z = g.uniform(-0.05, 0.05, N).astype(np.float16)
    return codes, s.view(np.uint16), z.view(np.uint16)


@pytest.mark.parametrize("seed,wide", [(0, False), (1, False), (2, True), (3, True), (4, True)])
def test_dequant_matches_exact_rational_emulation(seed, wide):
    codes, s, z = _case(seed, wide=wide)
    W = nf4.dequant_nf4(nf4.pack_codes(codes), codes.shape[1], s, z)
    t = nf4.nf4_table_f16()
    for n in range(codes.shape[0]):
        for k in range(codes.shape[1]):
            d = _r32(_f16val(t[codes[n, k]]) - _f16val(z[n]))
            w = _r32(d * _f16val(s[n]))
            want = _r16(w) if w is not None else None
            got = _f16val(W[n, k]) if np.isfinite(np.uint16(W[n, k]).view(np.float16)) else None
            assert got == want, (n, k)


def test_dequant_zero_point_absent_is_one_rounding():
    """z = 0: the fp32 product of two fp16 values is exact, so W is the
    single correct rounding of table[c] * s."""
    codes, s, _ = _case(5)
    W = nf4.dequant_nf4(nf4.pack_codes(codes), codes.shape[1], s)
    t = nf4.nf4_table_f16()
    for n in range(codes.shape[0]):
        for k in range(codes.shape[1]):
            assert _f16val(W[n, k]) == _r16(_f16val(t[codes[n, k]]) * _f16val(s[n]))


def test_dequant_unit_scale_is_the_table():
    codes = np.arange(16, dtype=np.uint8).reshape(1, 16).repeat(3, 0)
    one = np.full(3, 0x3C00, np.uint16)
    W = nf4.dequant_nf4(nf4.pack_codes(codes), 16, one)
    assert np.array_equal(W, np.tile(nf4.nf4_table_f16(), (3, 1)))


# -- GEMM -------------------------------------------------------------------


def _inputs(M, N, K, seed):
    g = np.random.default_rng(seed)
    A = g.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    codes, s, z = _case(seed + 100, N=N, K=K)
    return A, nf4.pack_codes(codes), s, z


def test_gemm_brute_force_exact_sums():
    M, N, K = 3, 5, 64
    A, Bp, s, z = _inputs(M, N, K, 0)
    C, S, absS = nf4.gemm_nf4_a16(A, Bp, s, z)
    W = nf4.dequant_nf4(Bp, K, s, z)
    for m in range(M):
        for n in range(N):
            prods = [float(_f16val(A[m, k]) * _f16val(W[n, k])) for k in range(K)]  # exact in float64
            exact = math.fsum(prods)
            assert abs(S[m, n] - exact) <= 1e-15 * absS[m, n] + 1e-300
            assert C[m, n] == np.float16(exact).view(np.uint16)
            assert abs(absS[m, n] - math.fsum(abs(p) for p in prods)) <= 1e-15 * absS[m, n]


def test_gemm_blocked_k_invariant():
    """Pallas page, blocked matmul: the sum of per-K-block products equals the
    full product (here to float64 rounding; each block's sum is exact-ish)."""
    M, N, K = 4, 6, 512
    A, Bp, s, z = _inputs(M, N, K, 1)
    _, S, absS = nf4.gemm_nf4_a16(A, Bp, s, z)
    for bk in (64, 128, 256):
        acc = np.zeros((M, N))
        for k0 in range(0, K, bk):
            _, Sb, _ = nf4.gemm_nf4_a16(A[:, k0:k0 + bk], Bp[:, k0 // 2:(k0 + bk) // 2], s, z)
            acc += Sb
        assert np.all(np.abs(acc - S) <= 1e-13 * absS + 1e-300)


def test_tolerance_covers_sequential_fp32_sum():
    """The bound of gemm_tolerance holds for a plain sequential fp32 sum of
    the exact products, rounded to fp16."""
    M, N, K = 8, 16, 4096
    A, Bp, s, z = _inputs(M, N, K, 2)
    _, S, absS = nf4.gemm_nf4_a16(A, Bp, s, z)
    tol = nf4.gemm_tolerance(S, absS, K)
    C_ref, _, _ = nf4.gemm_nf4_a16(A, Bp, s, z)
    Af = A.view(np.float16).astype(np.float32)
    Wf = nf4.dequant_nf4(Bp, K, s, z).view(np.float16).astype(np.float32)
    off_by_one = 0
    for m in range(M):
        for n in range(N):
            acc = np.float32(0)
            for p in (Af[m] * Wf[n]):  # products exact in fp32 (11 + 11 bits)
                acc = np.float32(acc + p)
            c = np.float16(acc)
            assert abs(c.astype(np.float64) - S[m, n]) <= tol[m, n]
            d = abs(int(c.view(np.int16)) - int(np.int16(C_ref[m, n].view(np.int16))))
            assert d <= 1  # same sign here; in practice one ulp at most
            off_by_one += d
    assert off_by_one <= M * N // 10


def test_library_table_matches_the_oracle():
    """The fp16 table compiled into the HIP library (written by its own
    generator, Newton's method on math.erf) equals the oracle's."""
    import os
    import re

    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "bit_mixed_precision_amd", "csrc", "nf4_table.h")
    text = open(path).read()
    body = text[text.index("kNf4TableF16"):]
    vals = [int(h, 16) for h in re.findall(r"0x([0-9A-Fa-f]{4})", body)]
    assert vals == nf4.nf4_table_f16().tolist()
