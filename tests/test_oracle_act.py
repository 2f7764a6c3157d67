"""Pins for the oracle's fused activation epilogue (JAX Pallas matmul page,
fused-activation section: the activation applied once to the wide result of
the last K step, then one downcast; BladeDISC page: GEMM + GELU fusion).

GELU is v * Phi(v) with Phi the standard normal CDF, evaluated as
erfc(-v / sqrt(2)) / 2.  Independent checks: mpmath's erfc at 50 significant
digits (arbitrary precision, no C library involved), scipy's erfc, printed
values of Phi, the identity GELU(-v) = GELU(v) - v, and for ReLU the exact
clamp of numpy's product."""
import mpmath
import numpy as np
import pytest
from scipy import special

from bit_mixed_precision_amd import synth


def _gelu_mp(v: float) -> float:
    """GELU at 50 significant digits, rounded once to double."""
    with mpmath.workdps(50):
        x = mpmath.mpf(v)
        return float(x * mpmath.erfc(-x / mpmath.sqrt(2)) / 2)


def test_gelu_matches_arbitrary_precision_erfc(oracle):
    """Close to the 50-digit value, also far into the negative tail where
    erfc is tiny (there 1 - erf would lose every digit).  Tolerance: the
    double argument -v/sqrt(2) carries a relative rounding error of about
    1e-16, which erfc's slope (-2x erfc(x) per unit of x) turns into a
    relative error of about 2x^2 1e-16 of the result, 1e-13 at v = -37; the
    result is then rounded to fp16 (relative 5e-4)."""
    for v in [-37.0, -25.0, -12.5, -8.0, -5.0, -1.7, -1e-3, -1e-30, 0.0, 1e-30, 2e-3, 0.5, 3.25, 9.0, 40.0]:
        ref = _gelu_mp(v)
        got = oracle.act(v, "gelu")
        assert got == pytest.approx(ref, rel=1e-12, abs=1e-320), v
        if abs(v) < 3:
            assert got == pytest.approx(ref, rel=2e-15, abs=1e-320), v
    # in the tail the value is nonzero and tiny: GELU(-12.5) ~ -1e-35
    assert -1e-34 < oracle.act(-12.5, "gelu") < -1e-36


def test_gelu_printed_cdf_values_and_symmetry(oracle):
    # standard normal CDF: Phi(1) = 0.8413447460685429..., Phi(2) = 0.9772498680518208...
    assert oracle.act(1.0, "gelu") == pytest.approx(0.8413447460685429, rel=1e-15)
    assert oracle.act(2.0, "gelu") == pytest.approx(2 * 0.9772498680518208, rel=1e-15)
    for v in [0.1, 0.77, 1.5, 4.0, 7.5]:
        assert oracle.act(-v, "gelu") == pytest.approx(oracle.act(v, "gelu") - v, rel=1e-12, abs=1e-15)


def test_relu_exact_and_identity(oracle):
    g = np.random.default_rng(41)
    acc = g.integers(-500_000, 500_000, (32, 48), dtype=np.int32)
    ws = synth.fp16_uniform(g, 48, 0.001, 0.01)
    xs = synth.fp16_uniform(g, 32, 0.05, 0.5)
    prod = acc.astype(np.float64) * ws.astype(np.float64)[None, :] * xs.astype(np.float64)[:, None]
    relu = np.maximum(prod, 0.0).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.dequant_act(acc, ws, xs, "relu"), relu)
    assert np.array_equal(oracle.dequant_act(acc, ws, xs, "none"), oracle.dequant2(acc, ws, xs))
    assert np.array_equal(oracle.dequant_act(acc, ws, None, "none"), oracle.dequant(acc, ws))


def test_gelu_fp16_outputs_match_scipy(oracle):
    g = np.random.default_rng(42)
    acc = g.integers(-3_000, 3_000, (64, 96), dtype=np.int32)
    acc[0, :4] = [0, -2500, 2500, -1]
    ws = synth.fp16_uniform(g, 96, 0.001, 0.004)
    v = acc.astype(np.float64) * ws.astype(np.float64)[None, :]
    ref = (0.5 * v * special.erfc(-v / np.sqrt(2.0))).astype(np.float16)
    got = oracle.dequant_act(acc, ws, None, "gelu")
    assert np.array_equal(got, ref.view(np.uint16))
    # large negative inputs: tiny results, down to the subnormal range of fp16
    accn = np.array([[-5000, -3000, -1000, -40000]], np.int32)
    wsn = np.full(4, 1e-3, np.float16)
    vn = accn.astype(np.float64) * wsn.astype(np.float64)
    refn = (0.5 * vn * special.erfc(-vn / np.sqrt(2.0))).astype(np.float16)
    gotn = oracle.dequant_act(accn, wsn, None, "gelu")
    assert np.array_equal(gotn, refn.view(np.uint16))
    assert 0 < abs(float(gotn.view(np.float16)[0, 0])) < 6.2e-5  # an fp16 subnormal


def test_bad_activation(oracle):
    with pytest.raises(KeyError):
        oracle.act(1.0, "tanh")
