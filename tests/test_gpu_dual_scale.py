"""GPU parity of the two-scale epilogue (per-token activation scale times
per-channel weight scale, BMINF page section 實現代碼分析2) against the
oracle, through the C ABI, on every kernel path; and the whole linear-layer
flow from fp16 activations (GPU quantization codes and scales bit-exact,
outputs within 1 fp16 ulp)."""
import numpy as np
import pytest

import oracle
from bit_mixed_precision_amd import synth
from gpu_util import assert_f16_within_1ulp, banner, f16_bits, need_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _weights(bits, N, K, seed):
    if bits == 8:
        _, Bv, ws = synth.w8a8_case(1, N, K, seed)
        return Bv, Bv, ws
    if bits == 4:
        _, Bv, ws = synth.w4a8_case(1, N, K, seed)
        return Bv, oracle.pack_int4(Bv), ws
    _, Bv, ws = synth.w2a8_case(1, N, K, seed, ternary=True)
    return Bv, oracle.pack_int2(Bv), ws


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("path,shape", [("gemv", (1, 100, 256)), ("gemv", (3, 37, 640)),
                                        ("stream", (5, 300, 384)), ("stream", (64, 130, 192)),
                                        ("tiled", (33, 100, 320)), ("tiled", (300, 260, 256)),
                                        ("tiled", (1000, 2100, 192)), ("tiled", (1030, 4100, 128)),
                                        ("auto", (4100, 4100, 64))])
def test_dual_scale_parity(dev, bits, path, shape):
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = shape
    banner(f"dual scale bits={bits} path={path} M={M} N={N} K={K}")
    g = np.random.default_rng(M + N + K + bits)
    A = synth.int8_uniform(g, (M, K))
    Bv, Bp, ws = _weights(bits, N, K, seed=M + N)
    xs = synth.fp16_uniform(g, M, 0.002, 0.05)
    xs[0] = np.float16(2.0 ** -24)  # a subnormal token scale
    C = bq.gemm_dual_scale(to_dev(A, dev), to_dev(Bp, dev), bits, to_dev(ws, dev), to_dev(xs, dev),
                           path=path)
    torch.cuda.synchronize()
    ref = oracle.dequant2(oracle.gemm_i32(A, Bv), ws, xs)
    assert_f16_within_1ulp(f16_bits(C), ref, f"dual scale w{bits} {path} {shape}")


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M", [1, 16, 64, 512])
def test_linear_flow_from_fp16(dev, bits, M):
    """fp16 activations X [M, K] -> per-token int8 (GPU vs oracle: codes and
    scales equal) -> two-scale GEMM with a quantized weight."""
    from bit_mixed_precision_amd import bq
    import torch

    N, K = 1024, 2048
    banner(f"linear flow bits={bits} M={M}")
    g = np.random.default_rng(M + bits)
    X = (g.standard_normal((M, K), np.float32) * np.float32(1.5)).astype(np.float16)
    Bv, Bp, ws = _weights(bits, N, K, seed=M)
    qx, sx = bq.quantize_rows(to_dev(X, dev))
    torch.cuda.synchronize()
    qx_ref, sx_ref = oracle.quantize_rows(X)
    assert np.array_equal(qx.cpu().numpy(), qx_ref)
    assert np.array_equal(f16_bits(sx), sx_ref)
    C = bq.linear(to_dev(X, dev), to_dev(Bp, dev), bits, to_dev(ws, dev))
    torch.cuda.synchronize()
    ref = oracle.gemm_wxa8_dequant2(qx_ref, Bp, ws, sx_ref, bits)
    assert_f16_within_1ulp(f16_bits(C), ref, f"linear flow w{bits} M={M}")


def test_dual_scale_errors(dev):
    from bit_mixed_precision_amd import bq
    import torch

    banner("dual scale errors")
    A = torch.zeros((4, 64), dtype=torch.int8, device=dev)
    B = torch.zeros((4, 64), dtype=torch.int8, device=dev)
    ws = torch.ones((4,), dtype=torch.float16, device=dev)
    with pytest.raises(ValueError):
        bq.gemm_dual_scale(A, B, 8, ws, torch.ones((3,), dtype=torch.float16, device=dev))
    # the GEMV path takes M <= 4
    A5 = torch.zeros((5, 64), dtype=torch.int8, device=dev)
    with pytest.raises(bq.BQError) as e:
        bq.gemm_dual_scale(A5, B, 8, ws, torch.ones((5,), dtype=torch.float16, device=dev), path="gemv")
    assert e.value.status == bq.BQ_ERR_SHAPE
