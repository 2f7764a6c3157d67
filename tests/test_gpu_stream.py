"""GPU parity of the streaming matrix-core GEMM (BQ_PATH_STREAM, M <= 256):
K split over a workgroup's wavefronts, chunk loads into per-wavefront LDS
buffers, partial tiles summed in LDS.  The shapes below select each of the
eight tile configurations (16x16 ... 64x64, by the library's traffic model)
with ragged M and N tails, K tails of half a 128-k chunk, K shorter than one
chunk per wavefront (idle wavefronts) and long K; int32 results must equal
the oracle's exactly, fp16 within one ulp of the correctly rounded value."""
import numpy as np
import pytest

import oracle
from bit_mixed_precision_amd import synth
from gpu_util import assert_f16_within_1ulp, banner, f16_bits, need_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _make(bits, M, N, K, seed):
    if bits == 8:
        A, Bv, s = synth.w8a8_case(M, N, K, seed)
        return A, Bv, Bv, s
    if bits == 4:
        A, Bv, s = synth.w4a8_case(M, N, K, seed)
        return A, Bv, oracle.pack_int4(Bv), s
    A, Bv, s = synth.w2a8_case(M, N, K, seed, ternary=(seed % 2 == 0))
    return A, Bv, oracle.pack_int2(Bv), s


# (M, N): 16x16 (3, 100); 16x32 (3, 4100); 16x64 (3, 8200); 32x32 (17, 4100);
# 32x64 (17, 8200); 64x32 (250, 1500, int8); 64x48 (33, 8200; 200, 3001
# int2); 64x64 (33, 12300)
MN = [(3, 100), (3, 4100), (3, 8200), (17, 4100), (17, 8200), (250, 1500), (33, 8200), (200, 3001),
      (33, 12300), (129, 700), (256, 333)]
KS = [64, 1088, 4160]


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("mn", MN)
@pytest.mark.parametrize("K", KS)
def test_stream_configs(dev, bits, mn, K):
    import torch

    from bit_mixed_precision_amd import bq

    M, N = mn
    banner(f"stream bits={bits} M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=M * 7 + N + K + bits)
    Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
    acc = bq.gemm(Ad, Bd, bits, None, path="stream")
    C = bq.gemm(Ad, Bd, bits, sd, path="stream")
    torch.cuda.synchronize()
    ref = oracle.gemm_i32(A, Bv)
    got = acc.cpu().numpy()
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        i, j = bad[0]
        raise AssertionError(f"w{bits} {M}x{N}x{K}: {len(bad)} int32 results differ; first at ({i}, {j}): "
                             f"got {got[i, j]} want {ref[i, j]}")
    assert_f16_within_1ulp(f16_bits(C), oracle.dequant(ref, s), f"w{bits} stream {M}x{N}x{K}")


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_stream_long_k_extremes(dev, bits):
    """K = 65536 (the ABI limit) with the extreme operands -127 x -8 / -2 /
    -128: every partial tile and their sum stay exact in int32."""
    import torch

    from bit_mixed_precision_amd import bq

    M, N, K = 40, 96, 65536
    banner(f"stream long K extremes bits={bits}")
    A = np.full((M, K), -127, np.int8)
    lo = {8: -128, 4: -8, 2: -2}[bits]
    Bv = np.full((N, K), lo, np.int8)
    Bp = Bv if bits == 8 else (oracle.pack_int4(Bv) if bits == 4 else oracle.pack_int2(Bv))
    acc = bq.gemm(to_dev(A, dev), to_dev(Bp, dev), bits, None, path="stream")
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i32(A, Bv))


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_stream_fused_epilogue(dev, bits):
    """The two-scale GELU epilogue on a mid-M streaming launch."""
    import torch

    from bit_mixed_precision_amd import bq

    M, N, K = 100, 700, 1088
    banner(f"stream fused epilogue bits={bits}")
    A, Bv, Bp, ws = _make(bits, M, N, K, seed=31 + bits)
    g = np.random.default_rng(bits)
    xs = synth.fp16_uniform(g, M, 0.002, 0.05)
    C = bq.gemm_act(to_dev(A, dev), to_dev(Bp, dev), bits, to_dev(ws, dev), to_dev(xs, dev), act="gelu",
                    path="stream")
    D = bq.gemm_dual_scale(to_dev(A, dev), to_dev(Bp, dev), bits, to_dev(ws, dev), to_dev(xs, dev),
                           path="stream")
    torch.cuda.synchronize()
    acc = oracle.gemm_i32(A, Bv)
    assert_f16_within_1ulp(f16_bits(C), oracle.dequant_act(acc, ws, xs, "gelu"), f"stream gelu w{bits}")
    assert_f16_within_1ulp(f16_bits(D), oracle.dequant2(acc, ws, xs), f"stream dual w{bits}")


def test_stream_batched_broadcast(dev):
    """The fused-QKV shape on the streaming path: three int4 weights, one
    activation of M = 96 broadcast to all three, two-scale epilogue."""
    import torch

    from bit_mixed_precision_amd import bq

    M, N, K = 96, 1000, 2048
    banner("stream batched broadcast")
    g = np.random.default_rng(77)
    A = synth.int8_uniform(g, (M, K))
    Bv = g.integers(-8, 7, (3, N, K), endpoint=True, dtype=np.int8)
    Bp = np.stack([oracle.pack_int4(b) for b in Bv])
    ws = np.stack([synth.fp16_uniform(g, N, 0.001, 0.01) for _ in range(3)])
    xs = synth.fp16_uniform(g, M, 0.01, 0.1)
    C = bq.gemm_batched(to_dev(A, dev), to_dev(Bp, dev), 4, to_dev(ws, dev), to_dev(xs, dev), path="stream")
    torch.cuda.synchronize()
    got = f16_bits(C)
    for z in range(3):
        ref = oracle.dequant2(oracle.gemm_i32(A, Bv[z]), ws[z], xs)
        assert_f16_within_1ulp(got[z], ref, f"stream batched z={z}")
