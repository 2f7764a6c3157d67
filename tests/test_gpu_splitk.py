"""GPU parity of bq_gemm_splitk: the tiled GEMM with K split over several
workgroups per output tile (64x64 tiles, at most 128 of them, K of at least
1024), exchanging int32 partial sums through a workspace the caller
allocates.  Each workgroup sums its share of K, the last to finish a tile
adds the others' partial sums and writes the tile.  Integer sums are exact,
so the results must equal the oracle's exactly (int32) or within 1 fp16 ulp,
whatever the split; the per-tile counters reset themselves, so repeated calls
and calls on two streams with their own workspaces must agree too, and a
workspace that is too small (or none) means no split, same results."""
import numpy as np
import pytest

import oracle
from bit_mixed_precision_amd import synth
from gpu_util import assert_f16_within_1ulp, banner, f16_bits, need_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _workspace(dev, M, N, K, bits):
    from bit_mixed_precision_amd import bq
    import torch

    n = bq.gemm_splitk_workspace_bytes(M, N, K, bits)
    assert n > 0, (M, N, K, bits)
    return torch.zeros(n, dtype=torch.uint8, device=dev)


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
    ws = _workspace(dev, M, N, K, bits)
    acc = bq.gemm_splitk(Ad, Bd, bits, None, ws)
    C = bq.gemm_splitk(Ad, Bd, bits, sd, ws)
    torch.cuda.synchronize()
    # every output against the oracle
    cols = np.arange(N)
    acc_ref = oracle.gemm_i32(A, np.ascontiguousarray(Bv[cols]))
    got = acc.cpu().numpy()[:, cols]
    assert np.array_equal(got, acc_ref), f"w{bits} {shape}: int32 results differ"
    assert_f16_within_1ulp(f16_bits(C)[:, cols], oracle.dequant(acc_ref, s[cols]), f"w{bits} {shape}")


def test_split_k_repeated_and_two_streams(dev):
    """Three calls in a row, then the same GEMM on two streams at once, each
    with its own workspace: the counters return to zero after every launch,
    so all results are identical."""
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = 64, 2048, 4096
    banner(f"split-K repeated / two streams M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(4, M, N, K, seed=5)
    Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
    ws = _workspace(dev, M, N, K, 4)
    first = bq.gemm_splitk(Ad, Bd, 4, sd, ws)
    for _ in range(2):
        again = bq.gemm_splitk(Ad, Bd, 4, sd, ws)
        torch.cuda.synchronize()
        assert torch.equal(again, first)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [_workspace(dev, M, N, K, 4) for _ in streams]
    outs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in streams]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for st, w, o in zip(streams, wss, outs):
            with torch.cuda.stream(st):
                bq.gemm_splitk(Ad, Bd, 4, sd, w, out=o)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, first)
    cols = np.arange(0, N, 5)
    ref = oracle.dequant(oracle.gemm_i32(A, np.ascontiguousarray(Bv[cols])), s[cols])
    assert_f16_within_1ulp(f16_bits(first)[:, cols], ref, "split-K w4 64x2048x4096")


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_split_k_small_or_no_workspace(dev, bits):
    """A workspace smaller than the shape needs, or none, runs K unsplit:
    the same exact results."""
    from bit_mixed_precision_amd import bq
    import torch

    M, N, K = 96, 640, 2048
    banner(f"split-K small / no workspace bits={bits}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=11 + bits)
    Ad, Bd = to_dev(A, dev), to_dev(Bp, dev)
    need = bq.gemm_splitk_workspace_bytes(M, N, K, bits)
    small = torch.zeros(need - 16, dtype=torch.uint8, device=dev)
    a = bq.gemm_splitk(Ad, Bd, bits, None, small)
    b = bq.gemm_splitk(Ad, Bd, bits, None, None)
    torch.cuda.synchronize()
    ref = oracle.gemm_i32(A, Bv)
    assert np.array_equal(a.cpu().numpy(), ref)
    assert np.array_equal(b.cpu().numpy(), ref)
    # the unused workspace was not touched
    assert int(small.count_nonzero()) == 0


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
    ws = _workspace(dev, M, N, K, 4)
    outs = [torch.empty((M, N), dtype=torch.int32, device=dev) for _ in range(40)]
    for o in outs:
        bq.gemm_splitk(Ad, Bd, 4, None, ws, out=o)
    torch.cuda.synchronize()
    ref = oracle.gemm_i32(A, Bv)
    for i, o in enumerate(outs):
        assert np.array_equal(o.cpu().numpy(), ref), f"launch {i} differs from the oracle"
