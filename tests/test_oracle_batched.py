"""Pins for the oracle's batched GEMM (BMINF page, section 實現代碼分析2: the
fused QKV weight (3, N, K) times one activation (1, M, K) broadcast over the
three weights, giving (3, M, N)).  Independent checks: numpy's exact int64
einsum over the batch, and numpy's float64 product rounded to float16 for
the epilogues."""
import numpy as np

from bit_mixed_precision_amd import synth


def test_batched_broadcast_int32_matches_einsum(oracle):
    g = np.random.default_rng(31)
    A = synth.int8_uniform(g, (9, 192))
    Bv = synth.int4_values(g, (3, 20, 192))
    Bp = np.stack([oracle.pack_int4(Bv[z]) for z in range(3)])
    ref = np.einsum("mk,bnk->bmn", A.astype(np.int64), Bv.astype(np.int64))
    assert np.array_equal(oracle.gemm_batched(A, Bp, 4), ref)


def test_batched_per_batch_a_and_scales(oracle):
    g = np.random.default_rng(32)
    A = synth.int8_uniform(g, (2, 5, 128))
    Bv = synth.ternary_values(g, (2, 7, 128))
    Bp = np.stack([oracle.pack_int2(Bv[z]) for z in range(2)])
    ws = np.stack([synth.fp16_uniform(g, 7, 0.5, 2.0) for _ in range(2)])
    xs = synth.fp16_uniform(g, 5, 0.01, 0.1)
    acc = np.einsum("bmk,bnk->bmn", A.astype(np.int64), Bv.astype(np.int64)).astype(np.float64)
    ref1 = (acc * ws.astype(np.float64)[:, None, :]).astype(np.float16)
    ref2 = (acc * ws.astype(np.float64)[:, None, :] * xs.astype(np.float64)[None, :, None]).astype(np.float16)
    assert np.array_equal(oracle.gemm_batched(A, Bp, 2, ws), ref1.view(np.uint16))
    assert np.array_equal(oracle.gemm_batched(A, Bp, 2, ws, xs), ref2.view(np.uint16))
