"""GPU parity of the batched GEMM (one launch over a batch of weights; the
fused-QKV shape of the BMINF page, section 實現代碼分析2: a (3, N, K) weight
times one (1, M, K) activation broadcast over the three weights) against the
oracle, through the C ABI, on every kernel path, with int32, one-scale and
two-scale outputs, broadcast and per-batch activations, and padded strides."""
import ctypes

import numpy as np
import pytest

import oracle
from bit_mixed_precision_amd import synth
from gpu_util import assert_f16_within_1ulp, banner, f16_bits, need_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _case(bits, batch, M, N, K, seed, shared_a=True):
    g = np.random.default_rng(seed)
    A = synth.int8_uniform(g, (M, K) if shared_a else (batch, M, K))
    if bits == 8:
        Bv = synth.int8_uniform(g, (batch, N, K))
        Bp = Bv
    elif bits == 4:
        Bv = synth.int4_values(g, (batch, N, K))
        Bp = np.stack([oracle.pack_int4(Bv[z]) for z in range(batch)])
    else:
        Bv = synth.ternary_values(g, (batch, N, K))
        Bp = np.stack([oracle.pack_int2(Bv[z]) for z in range(batch)])
    ws = np.stack([synth.fp16_uniform(g, N, 0.001, 0.01) for _ in range(batch)])
    xs = synth.fp16_uniform(g, M, 0.01, 0.1)
    return A, Bp, ws, xs


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("path,shape", [("gemv", (3, 1, 96, 256)), ("stream", (3, 17, 200, 384)),
                                        ("tiled", (3, 64, 320, 256)), ("tiled", (2, 300, 136, 192)),
                                        ("auto", (3, 1030, 1040, 128))])
def test_batched_broadcast_parity(dev, bits, path, shape):
    from bit_mixed_precision_amd import bq
    import torch

    batch, M, N, K = shape
    banner(f"batched bits={bits} path={path} batch={batch} M={M} N={N} K={K}")
    A, Bp, ws, xs = _case(bits, batch, M, N, K, seed=sum(shape) + bits)
    Ad, Bd, wsd, xsd = to_dev(A, dev), to_dev(Bp, dev), to_dev(ws, dev), to_dev(xs, dev)
    acc = bq.gemm_batched(Ad, Bd, bits, path=path)
    C1 = bq.gemm_batched(Ad, Bd, bits, wsd, path=path)
    C2 = bq.gemm_batched(Ad, Bd, bits, wsd, xsd, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_batched(A, Bp, bits))
    assert_f16_within_1ulp(f16_bits(C1), oracle.gemm_batched(A, Bp, bits, ws), f"batched w{bits} {path}")
    assert_f16_within_1ulp(f16_bits(C2), oracle.gemm_batched(A, Bp, bits, ws, xs), f"batched2 w{bits} {path}")


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_batched_largest_tile_configuration(dev, bits):
    """Two weights of 4104 x 128 behind one 4100 x 128 activation: 289 tiles of
    256 x 256 per weight, so the batch runs the largest tile configuration with
    M and N tails (N a multiple of 8, so that each weight's scale row starts
    16-byte aligned); int32, one- and two-scale outputs on sampled rows and
    columns of both weights, the ragged last tile row and column included."""
    from bit_mixed_precision_amd import bq
    import torch

    batch, M, N, K = 2, 4100, 4104, 128
    banner(f"batched largest tiles bits={bits} batch={batch} M={M} N={N} K={K}")
    A, Bp, ws, xs = _case(bits, batch, M, N, K, seed=41 + bits)
    Ad, Bd, wsd, xsd = to_dev(A, dev), to_dev(Bp, dev), to_dev(ws, dev), to_dev(xs, dev)
    acc = bq.gemm_batched(Ad, Bd, bits).cpu().numpy()
    C1 = f16_bits(bq.gemm_batched(Ad, Bd, bits, wsd))
    C2 = f16_bits(bq.gemm_batched(Ad, Bd, bits, wsd, xsd))
    g = np.random.default_rng(bits)
    rows = np.unique(np.concatenate([g.choice(M, 48, replace=False), np.arange(M - 8, M), [0]]))
    cols = np.unique(np.concatenate([g.choice(N, 512, replace=False), np.arange(N - 40, N), [0]]))
    A_s, B_s, ws_s = np.ascontiguousarray(A[rows]), np.ascontiguousarray(Bp[:, cols]), np.ascontiguousarray(ws[:, cols])
    sel = np.ix_(np.arange(batch), rows, cols)
    assert np.array_equal(acc[sel], oracle.gemm_batched(A_s, B_s, bits))
    assert_f16_within_1ulp(C1[sel], oracle.gemm_batched(A_s, B_s, bits, ws_s), f"batched large w{bits}")
    assert_f16_within_1ulp(C2[sel], oracle.gemm_batched(A_s, B_s, bits, ws_s, xs[rows]), f"batched2 large w{bits}")


@pytest.mark.parametrize("bits", [8, 4])
def test_batched_per_batch_activations(dev, bits):
    from bit_mixed_precision_amd import bq
    import torch

    banner(f"batched per-batch A bits={bits}")
    A, Bp, ws, _ = _case(bits, 4, 70, 264, 320, seed=7 + bits, shared_a=False)
    C = bq.gemm_batched(to_dev(A, dev), to_dev(Bp, dev), bits, to_dev(ws, dev))
    torch.cuda.synchronize()
    assert_f16_within_1ulp(f16_bits(C), oracle.gemm_batched(A, Bp, bits, ws), "batched per-batch A")


def test_batched_padded_strides_via_abi(dev):
    """Strides larger than the matrices (padding between batches) through the
    C call directly; the padding of the output is left untouched."""
    from bit_mixed_precision_amd import bq
    import torch

    banner("batched padded strides")
    batch, M, N, K = 3, 20, 40, 128
    A, Bp, ws, _ = _case(8, batch, M, N, K, seed=3)
    padB, padS, padC = N * K + 64, N + 8, M * N + 40
    Bbuf = torch.zeros(batch * padB, dtype=torch.int8, device=dev)
    Sbuf = torch.zeros(batch * padS, dtype=torch.float16, device=dev)
    Cbuf = torch.full((batch * padC,), -1.0, dtype=torch.float16, device=dev)
    for z in range(batch):
        Bbuf[z * padB: z * padB + N * K] = to_dev(Bp[z].reshape(-1), dev)
        Sbuf[z * padS: z * padS + N] = to_dev(ws[z], dev)
    Ad = to_dev(A, dev)
    st = bq.lib().bq_gemm_batched(Ad.data_ptr(), 0, Bbuf.data_ptr(), padB, 8, Sbuf.data_ptr(), padS,
                                  None, Cbuf.data_ptr(), padC, batch, M, N, K, 0,
                                  ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    ref = oracle.gemm_batched(A, Bp, 8, ws)
    got = f16_bits(Cbuf)
    for z in range(batch):
        assert_f16_within_1ulp(got[z * padC: z * padC + M * N].reshape(M, N), ref[z], f"padded z={z}")
        assert np.all(got[z * padC + M * N: (z + 1) * padC] == np.float16(-1.0).view(np.uint16))


def test_batched_errors(dev):
    from bit_mixed_precision_amd import bq
    import torch

    banner("batched errors")
    L = bq.lib()
    A = torch.zeros((4, 64), dtype=torch.int8, device=dev)
    B = torch.zeros((2, 8, 64), dtype=torch.int8, device=dev)
    C = torch.zeros((2, 4, 8), dtype=torch.int32, device=dev)
    S = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    # overlapping outputs, negative stride, misaligned stride, batch limit
    assert L.bq_gemm_batched(A.data_ptr(), 0, B.data_ptr(), 512, 8, None, 0, None, C.data_ptr(), 16,
                             2, 4, 8, 64, 0, S) == bq.BQ_ERR_SHAPE
    assert L.bq_gemm_batched(A.data_ptr(), -256, B.data_ptr(), 512, 8, None, 0, None, C.data_ptr(), 32,
                             2, 4, 8, 64, 0, S) == bq.BQ_ERR_SHAPE
    assert L.bq_gemm_batched(A.data_ptr(), 0, B.data_ptr(), 520, 8, None, 0, None, C.data_ptr(), 32,
                             2, 4, 8, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm_batched(A.data_ptr(), 0, B.data_ptr(), 512, 8, None, 0, None, C.data_ptr(), 32,
                             65536, 4, 8, 64, 0, S) == bq.BQ_ERR_SHAPE
    # fp16 outputs: a weight-scale stride or an output stride that is not a
    # multiple of 8 elements leaves the next batch's row misaligned
    W = torch.ones((2, 16), dtype=torch.float16, device=dev)
    H = torch.zeros((2, 40), dtype=torch.float16, device=dev)
    assert L.bq_gemm_batched(A.data_ptr(), 0, B.data_ptr(), 512, 8, W.data_ptr(), 4, None, H.data_ptr(), 40,
                             2, 4, 8, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm_batched(A.data_ptr(), 0, B.data_ptr(), 512, 8, W.data_ptr(), 8, None, H.data_ptr(), 36,
                             2, 4, 8, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm_batched(A.data_ptr(), 0, B.data_ptr(), 512, 8, W.data_ptr(), 8, None, H.data_ptr(), 40,
                             2, 4, 8, 64, 0, S) == bq.BQ_OK
    torch.cuda.synchronize()
    # batch 0 is a no-op
    assert L.bq_gemm_batched(None, 0, None, 0, 8, None, 0, None, None, 0, 0, 4, 8, 64, 0, S) == bq.BQ_OK
