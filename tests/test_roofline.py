"""Pins the work/traffic model to the worked values printed on the Pallas
matmul page (tests/golden/pallas_roofline.txt)."""
import os

import pytest

from bit_mixed_precision_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pallas_roofline.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_pallas_worked_values():
    """With every operand at one width the model is the page's: 2 m k n
    operations and (m k + k n + m n) * itemsize bytes at 1024^3 in f32."""
    g = _golden()
    ops = roofline.gemm_ops(1024, 1024, 1024)
    b32 = roofline.operand_bytes(1024, 1024, 1024, 4, 32, 4)
    b16 = roofline.operand_bytes(1024, 1024, 1024, 2, 16, 2)
    assert ops == g["matmul_flops_1024_1024_1024"]
    assert b32 == g["matmul_membw_1024_1024_1024_f32"]
    assert ops / b32 == pytest.approx(g["intensity_1024_f32_approx"], abs=0.05)
    assert ops / b16 == pytest.approx(g["intensity_1024_bf16_approx"], abs=0.5)
    assert g["v5e_flops"] / g["v5e_membw"] == pytest.approx(g["v5e_ridge_approx"], abs=0.05)
    # square f32 matmul crosses the v5e ridge at m = k = n ~ 1440: 2m^3 / 12m^2 = 240
    m = g["square_crossover_f32"]
    assert 2 * m ** 3 / (12 * m ** 2) == pytest.approx(240, abs=0.1)


def test_mixed_width_bytes():
    # W4A8 GEMV at M=1, N=K=4096: A 4096 + B 4096*4096/2 + scale 8192 + out 8192
    assert roofline.gemm_bytes(1, 4096, 4096, 4) == 4096 + 8388608 + 8192 + 8192
    # reduces to the page's model when every operand has the same width
    assert roofline.gemm_bytes(64, 32, 128, 8, out="i32") == 64 * 128 + 32 * 128 + 4 * 64 * 32
    assert roofline.quantize_bytes(12288, 4096) == 151019520
    assert roofline.pack_bytes(4096, 4096, 4) == 4096 * 4096 * 3 // 2
    assert roofline.gemm_ops(4096, 4096, 4096) == 137438953472
