"""GPU parity of the tiled GEMM when K is split over several workgroups per
output tile (64x64 tiles, at most 128 of them, K of at least 1024): each
workgroup sums its share of K, the last to finish a tile adds the others'
partial sums and writes the tile.  Integer sums are exact, so the results
must equal the oracle's exactly (int32) or within 1 fp16 ulp, whatever the
split; the per-tile counters reset themselves, so repeated calls and calls on
two streams must agree too."""
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
    A, Bv, s = synth.w2a8_case(M, N, K, seed, ternary=True)
    return A, Bv, oracle.pack_int2(Bv), s


# (M, N, K): tiles x parts chosen by the library, e.g. 1 x 8, 16 x 7 with
# a 3-stage last part and a K tail, 65 x 2 with a ragged N, 20 x 8, 64 x 4
SPLIT_SHAPES = [(3, 40, 8192), (128, 512, 4160), (33, 4100, 1024), (200, 300, 8192),
                (64, 4096, 4096)]


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_split_k_parity(dev, bits, shape):
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = shape
    banner(f"split-K bits={bits} M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=M + N + K + bits)
    Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
    acc = bq.gemm(Ad, Bd, bits, None, path="tiled")
    C = bq.gemm(Ad, Bd, bits, sd, path="tiled")
    torch.cuda.synchronize()
    # every row against the oracle on a sample of columns (all of them when
    # N is small), plus the last column (the ragged N tail)
    cols = np.arange(N) if N <= 512 else np.unique(np.r_[np.arange(0, N, 7), N - 1])
    acc_ref = oracle.gemm_i32(A, np.ascontiguousarray(Bv[cols]))
    got = acc.cpu().numpy()[:, cols]
    assert np.array_equal(got, acc_ref), f"w{bits} {shape}: int32 results differ"
    assert_f16_within_1ulp(f16_bits(C)[:, cols], oracle.dequant(acc_ref, s[cols]), f"w{bits} {shape}")


def test_split_k_repeated_and_two_streams(dev):
    """Three calls in a row, then the same GEMM on two streams at once: the
    counters return to zero after every launch and each stream has its own
    workspace, so all results are identical."""
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = 64, 2048, 4096
    banner(f"split-K repeated / two streams M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(4, M, N, K, seed=5)
    Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
    first = bq.gemm(Ad, Bd, 4, sd, path="tiled")
    for _ in range(2):
        again = bq.gemm(Ad, Bd, 4, sd, path="tiled")
        torch.cuda.synchronize()
        assert torch.equal(again, first)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in streams]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for st, o in zip(streams, outs):
            with torch.cuda.stream(st):
                bq.gemm(Ad, Bd, 4, sd, out=o, path="tiled")
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, first)
    cols = np.arange(0, N, 5)
    ref = oracle.dequant(oracle.gemm_i32(A, np.ascontiguousarray(Bv[cols])), s[cols])
    assert_f16_within_1ulp(f16_bits(first)[:, cols], ref, "split-K w4 64x2048x4096")


@pytest.mark.parametrize("bits", [8, 4])
def test_split_k_fused_epilogue(dev, bits):
    """The two-scale GELU epilogue on a split tile (the last workgroup runs it
    on the summed accumulators)."""
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = 96, 640, 2048
    banner(f"split-K fused epilogue bits={bits}")
    A, Bv, Bp, ws = _make(bits, M, N, K, seed=11 + bits)
    g = np.random.default_rng(bits)
    xs = synth.fp16_uniform(g, M, 0.002, 0.05)
    C = bq.gemm_act(to_dev(A, dev), to_dev(Bp, dev), bits, to_dev(ws, dev), to_dev(xs, dev),
                    act="gelu", path="tiled")
    torch.cuda.synchronize()
    ref = oracle.dequant_act(oracle.gemm_i32(A, Bv), ws, xs, "gelu")
    assert_f16_within_1ulp(f16_bits(C), ref, f"split-K gelu w{bits}")


@pytest.mark.parametrize("shape", [(3, 40, 8192), (200, 300, 8192), (100, 200, 1088)])
def test_split_k_many_launches_agree(dev, shape):
    """Forty launches in a row (1 tile x 8 parts and 20 x 8, whose parts run
    on different XCDs since the tile count is not a multiple of 8; 8 x 2 with
    a K tail): every int32 result equals the oracle's, so no launch read a
    partial sum before it was complete."""
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = shape
    banner(f"split-K 40 launches M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(4, M, N, K, seed=7)
    Ad, Bd = to_dev(A, dev), to_dev(Bp, dev)
    outs = [torch.empty((M, N), dtype=torch.int32, device=dev) for _ in range(40)]
    for o in outs:
        bq.gemm(Ad, Bd, 4, None, out=o, path="tiled")
    torch.cuda.synchronize()
    ref = oracle.gemm_i32(A, Bv)
    for i, o in enumerate(outs):
        assert np.array_equal(o.cpu().numpy(), ref), f"launch {i} differs from the oracle"
