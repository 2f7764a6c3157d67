"""Pins for the oracle's two-scale epilogue of a linear layer whose input is
quantized per token (BMINF page, section 實現代碼分析2, PartialAttention
forward: quantize(hidden, axis=1) gives int8 codes and one fp16 scale per
token; igemm multiplies them with the int8 weight; elementwise_copy_scale
computes out0 = in0 * in1 * in2 with the weight scale of the output channel
and the scale of the token).

Independent checks: numpy's float64 product (exact for an int32 and two fp16
factors) rounded by numpy's float64 -> float16 conversion; exact rational
arithmetic with ties to even; the reduction to the one-scale epilogue when
every token scale is 1; and, for the whole flow from fp16 activations and
weights, the error bound that the two per-row quantizations allow.
"""
from fractions import Fraction

import numpy as np
import pytest

from bit_mixed_precision_amd import synth


def test_dequant2_matches_numpy_rounding(oracle):
    g = np.random.default_rng(21)
    M, N = 48, 80
    acc = g.integers(-3_000_000, 3_000_000, (M, N), dtype=np.int32)
    acc[0, :6] = [0, 1, -1, 2**31 - 1, -2**31, 65519]
    ws = synth.fp16_uniform(g, N, 0.0005, 0.02)
    xs = synth.fp16_uniform(g, M, 0.001, 0.05)
    ws[:6] = 1.0
    xs[0] = 1.0
    xs[1] = np.float16(2.0 ** -24)  # smallest subnormal token scale
    with np.errstate(over="ignore"):
        ref = (acc.astype(np.float64) * ws.astype(np.float64)[None, :]
               * xs.astype(np.float64)[:, None]).astype(np.float16)
    got = oracle.dequant2(acc, ws, xs)
    assert np.array_equal(got, ref.view(np.uint16))
    assert got[0, 3] == 0x7C00 and got[0, 4] == 0xFC00  # +-inf past 65520
    assert got[0, 5] == np.float16(65504).view(np.uint16)


def test_dequant2_unit_token_scale_is_dequant(oracle):
    g = np.random.default_rng(22)
    acc = g.integers(-200_000, 200_000, (16, 40), dtype=np.int32)
    ws = synth.fp16_uniform(g, 40, 0.001, 0.01)
    ones = np.ones(16, np.float16)
    assert np.array_equal(oracle.dequant2(acc, ws, ones), oracle.dequant(acc, ws))


def test_dequant2_exact_fraction_sample(oracle):
    g = np.random.default_rng(23)
    acc = g.integers(-90_000, 90_000, (6, 32), dtype=np.int32)
    ws = synth.fp16_uniform(g, 32, 0.001, 0.01)
    xs = synth.fp16_uniform(g, 6, 0.01, 0.2)
    got = oracle.dequant2(acc, ws, xs)
    for i in range(6):
        for j in range(32):
            exact = Fraction(int(acc[i, j])) * Fraction(float(ws[j])) * Fraction(float(xs[i]))
            bits = int(got[i, j])
            v = Fraction(float(np.uint16(bits).view(np.float16)))
            for nb in (bits - 1, bits + 1):
                w = Fraction(float(np.uint16(nb).view(np.float16)))
                assert abs(w - exact) > abs(v - exact) or (
                    abs(w - exact) == abs(v - exact) and bits % 2 == 0)


def test_per_token_flow_error_bound(oracle):
    """fp16 X [M,K] and W [N,K] quantized per row, integer GEMM, two-scale
    epilogue: the result is X W^T up to the quantization error,
    |x - qx sx| <= sx/2 and |w - qw sw| <= sw/2, plus the final fp16 rounding.
    A scale applied along the wrong axis breaks the bound by orders of
    magnitude."""
    g = np.random.default_rng(24)
    M, N, K = 12, 40, 256
    X = (g.standard_normal((M, K), np.float32) * np.float32(2.0)).astype(np.float16)
    X[3] *= np.float16(0.01)  # a token with a much smaller range
    W = (g.standard_normal((N, K), np.float32) * np.float32(0.02)).astype(np.float16)
    qx, sx = oracle.quantize_rows(X)
    qw, sw = oracle.quantize_rows(W)
    out = oracle.gemm_wxa8_dequant2(qx, qw, sw, sx, 8).view(np.float16).astype(np.float64)
    x = X.astype(np.float64)
    w = W.astype(np.float64)
    sxf = sx.view(np.float16).astype(np.float64)
    swf = sw.view(np.float16).astype(np.float64)
    ref = x @ w.T
    bound = (np.abs(x).sum(1)[:, None] * swf[None, :] / 2 + np.abs(w).sum(1)[None, :] * sxf[:, None] / 2
             + K * sxf[:, None] * swf[None, :] / 4)
    bound += np.abs(ref) * 2.0 ** -11 + 2.0 ** -24  # final fp16 rounding
    assert np.all(np.abs(out - ref) <= bound)
    # the bound is tight enough to see token scales applied to the wrong rows
    perm = np.roll(np.arange(M), 1)
    wrong = oracle.gemm_wxa8_dequant2(qx, qw, sw, sx[perm], 8).view(np.float16).astype(np.float64)
    assert not np.all(np.abs(wrong - ref) <= bound)


def test_dequant2_shape_errors(oracle):
    acc = np.zeros((3, 4), np.int32)
    with pytest.raises(ValueError):
        oracle.dequant2(acc, np.ones(3, np.float16), np.ones(3, np.float16))
    with pytest.raises(ValueError):
        oracle.dequant2(acc, np.ones(4, np.float16), np.ones(4, np.float16))
