"""GPU parity of the fused activation epilogue (JAX Pallas matmul page,
fused-activation section; BladeDISC page, GEMM + GELU) against the oracle,
through the C ABI, on every kernel path and tile configuration, with and
without the per-token scale; fp16 outputs within 1 ulp of the correctly
rounded act(acc * w_scale * x_scale)."""
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


@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("path,shape", [("gemv", (2, 100, 256)), ("stream", (20, 130, 320)),
                                        ("tiled", (100, 200, 1088)), ("tiled", (1000, 2100, 192)),
                                        ("tiled", (1030, 4100, 128)), ("auto", (4100, 4100, 64))])
def test_act_parity(dev, act, bits, path, shape):
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = shape
    banner(f"act={act} bits={bits} path={path} M={M} N={N} K={K}")
    g = np.random.default_rng(M + N + K + bits)
    A = synth.int8_uniform(g, (M, K))
    Bv, Bp, ws = _weights(bits, N, K, seed=M + N)
    # scales that put the dequantized values across GELU's curved range [-6, 6]
    ws = (ws.astype(np.float32) * np.float32(4.0 / np.sqrt(K))).astype(np.float16)
    xs = synth.fp16_uniform(g, M, 0.25, 1.0)
    acc = oracle.gemm_i32(A, Bv)
    Ad, Bd, wsd, xsd = to_dev(A, dev), to_dev(Bp, dev), to_dev(ws, dev), to_dev(xs, dev)
    C1 = bq.gemm_act(Ad, Bd, bits, wsd, None, act=act, path=path)
    C2 = bq.gemm_act(Ad, Bd, bits, wsd, xsd, act=act, path=path)
    torch.cuda.synchronize()
    assert_f16_within_1ulp(f16_bits(C1), oracle.dequant_act(acc, ws, None, act), f"{act} w{bits} {path}")
    assert_f16_within_1ulp(f16_bits(C2), oracle.dequant_act(acc, ws, xs, act), f"{act}+xs w{bits} {path}")


def test_linear_gelu_flow(dev):
    from bit_mixed_precision_amd import bq
    import torch

    banner("linear flow with GELU")
    M, N, K = 64, 1024, 2048
    g = np.random.default_rng(5)
    X = (g.standard_normal((M, K), np.float32)).astype(np.float16)
    Bv, Bp, ws = _weights(8, N, K, seed=9)
    C = bq.linear(to_dev(X, dev), to_dev(Bp, dev), 8, to_dev(ws, dev), act="gelu")
    torch.cuda.synchronize()
    qx, sx = oracle.quantize_rows(X)
    ref = oracle.dequant_act(oracle.gemm_i32(qx, Bv), ws, sx, "gelu")
    assert_f16_within_1ulp(f16_bits(C), ref, "linear gelu")


@pytest.mark.parametrize("path", ["tiled", "stream", "gemv"])
def test_gelu_dense_sweep(dev, path):
    """GELU over a dense grid of dequantized values: acc[m, n] = a_m for
    a = -127..127 (A[m, 0] = a_m, B[n, 0] = 1, everything else 0) and 256
    weight scales from 2^-8 to 2^-3, so v = a_m * s_n covers [-16, 16] with
    steps down to 2^-8; fp16 outputs within 1 ulp of the exact GELU."""
    from bit_mixed_precision_amd import bq
    import torch

    banner(f"gelu dense sweep path={path}")
    a = np.arange(-127, 128, dtype=np.int8)
    if path == "stream":
        a = a[::4][:64]
    elif path == "gemv":
        a = np.array([-127, -3, 5, 126], dtype=np.int8)
    M, N, K = len(a), 256, 64
    A = np.zeros((M, K), np.int8)
    A[:, 0] = a
    Bv = np.zeros((N, K), np.int8)
    Bv[:, 0] = 1
    ws = np.exp2(np.linspace(-8.0, -3.0, N)).astype(np.float16)
    C = bq.gemm_act(to_dev(A, dev), to_dev(Bv, dev), 8, to_dev(ws, dev), None, act="gelu", path=path)
    torch.cuda.synchronize()
    ref = oracle.dequant_act(oracle.gemm_i32(A, Bv), ws, None, "gelu")
    assert_f16_within_1ulp(f16_bits(C), ref, f"gelu sweep {path}")


_PP_CACHE = {}


@pytest.mark.parametrize("K", [1024, 1088])
@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
def test_pingpong_fused_epilogue_full(dev, act, K):
    """W4A8 at M = N = 4096 runs the 256 x 256 ping-pong kernel; with K =
    1024 (eight stages) and 1088 (a half stage past the last whole one) the
    fused epilogue (weight scale, optional per-token scale, activation) is
    checked on every output after a multi-stage K loop, against the oracle."""
    from bit_mixed_precision_amd import bq
    import torch

    M = N = 4096
    banner(f"pingpong fused act={act} M={M} N={N} K={K}")
    if K not in _PP_CACHE:
        g = np.random.default_rng(K)
        A = synth.int8_uniform(g, (M, K))
        Bv, Bp, ws = _weights(4, N, K, seed=K + 3)
        ws = (ws.astype(np.float32) * np.float32(4.0 / np.sqrt(K))).astype(np.float16)
        xs = synth.fp16_uniform(g, M, 0.25, 1.0)
        _PP_CACHE.clear()
        _PP_CACHE[K] = (A, Bp, ws, xs, oracle.gemm_i32(A, Bv))
    A, Bp, ws, xs, acc = _PP_CACHE[K]
    Ad, Bd, wsd, xsd = to_dev(A, dev), to_dev(Bp, dev), to_dev(ws, dev), to_dev(xs, dev)
    C1 = bq.gemm_act(Ad, Bd, 4, wsd, None, act=act)
    C2 = bq.gemm_act(Ad, Bd, 4, wsd, xsd, act=act)
    torch.cuda.synchronize()
    assert_f16_within_1ulp(f16_bits(C1), oracle.dequant_act(acc, ws, None, act), f"pp {act} K={K}")
    assert_f16_within_1ulp(f16_bits(C2), oracle.dequant_act(acc, ws, xs, act), f"pp {act}+xs K={K}")
