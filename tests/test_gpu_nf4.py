"""GPU parity of the W4A16 GEMM with NF4 weight codes (bq_gemm_nf4_a16)
against the oracle (oracle/nf4.py), through the C ABI.

* Exact cases: integer activations |a| <= amax, no zero point, scale 2^-7.
  The fp16 table values are multiples of 2^-14, so every product is a
  multiple of L = 2^-21 and every partial sum is at most K amax 2^-7 =
  K amax 2^14 L <= 2^24 L in magnitude (K amax <= 1024): an integer multiple
  of L below 2^24 L, exact in fp32.  So any accumulation order is exact and
  the fp16 output must equal the oracle's bit for bit.  These run on every
  tile configuration (64 x 64 with and without the K split, 128 x 128,
  256 x 256).
* Random cases (normal activations, scales in [0.001, 0.01], zero points in
  [-0.05, 0.05]): every output within the oracle's fp32-accumulation bound
  (gemm_tolerance), and nearly all within one fp16 ulp of the exact sum."""
import numpy as np
import pytest

from oracle import nf4
from gpu_util import banner, f16_bits, need_gpu, ord16, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _run(dev, A, Bp, s, z):
    from bit_mixed_precision_amd import bq
    import torch

    C = bq.gemm_nf4_a16(to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev),
                        None if z is None else to_dev(z, dev))
    torch.cuda.synchronize()
    return f16_bits(C)


# (M, N, K, amax): 64x64 without split, 64x64 with K split over 4 parts
# (64 and 4 tiles), 64x64 4-stage (>= 512 tiles), 128x128, 256x256, with
# ragged M and N
EXACT_SHAPES = [(1, 200, 256, 3), (33, 130, 256, 3), (1, 4096, 1024, 1), (64, 256, 1024, 1),
                (1100, 1900, 256, 3), (1030, 4100, 256, 3), (4100, 4100, 256, 3)]


@pytest.mark.parametrize("shape", EXACT_SHAPES)
def test_nf4_exact_integer_activations(dev, shape):
    M, N, K, amax = shape
    banner(f"nf4 exact M={M} N={N} K={K}")
    g = np.random.default_rng(M + N)
    A = g.integers(-amax, amax + 1, (M, K)).astype(np.float16).view(np.uint16)
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    Bp = nf4.pack_codes(codes)
    s = np.full(N, np.float16(2.0 ** -7)).view(np.uint16)
    C = _run(dev, A, Bp, s, None)
    C_ref, _, _ = nf4.gemm_nf4_a16(A, Bp, s)
    assert np.array_equal(C, C_ref), f"{int((C != C_ref).sum())} of {C.size} outputs differ"


def _random_case(M, N, K, seed, zero=True):
    g = np.random.default_rng(seed)
    A = g.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    s = g.uniform(0.001, 0.01, N).astype(np.float16).view(np.uint16)
    z = g.uniform(-0.05, 0.05, N).astype(np.float16).view(np.uint16) if zero else None
    return A, nf4.pack_codes(codes), s, z


RANDOM_SHAPES = [(1, 4096, 4096), (1, 11008, 4096), (2, 301, 512), (3, 777, 64), (4, 130, 65536),
                 (5, 64, 128), (16, 256, 256), (64, 4096, 4096), (300, 260, 1024), (300, 2000, 4096),
                 (1030, 1100, 512), (4096, 4096, 512)]


@pytest.mark.parametrize("shape", RANDOM_SHAPES)
@pytest.mark.parametrize("zero", [True, False])
def test_nf4_random_within_fp32_bound(dev, shape, zero):
    M, N, K = shape
    banner(f"nf4 random M={M} N={N} K={K} zero={zero}")
    A, Bp, s, z = _random_case(M, N, K, seed=M + N + K, zero=zero)
    C = _run(dev, A, Bp, s, z)
    # all rows for small M, else every 17th row (plus the last); all columns
    rows = np.arange(M) if M <= 64 else np.unique(np.r_[np.arange(0, M, 17), M - 1])
    _, S, absS = nf4.gemm_nf4_a16(A[rows], Bp, s, z)
    tol = nf4.gemm_tolerance(S, absS, K)
    got = C[rows].view(np.float16).astype(np.float64)
    err = np.abs(got - S)
    assert np.all(np.isfinite(got))
    bad = err > tol
    assert not bad.any(), f"{int(bad.sum())} outputs outside the fp32 bound; worst {float((err / tol).max()):.2f}x"
    # in practice the fp32 sums are much closer: the correctly rounded fp16
    # of the exact sum, or one ulp away, for all but a few outputs (those
    # near zero, where an fp16 ulp is tiny against the fp32 error)
    C_ref = S.astype(np.float16).view(np.uint16)
    d = np.abs(ord16(C[rows]) - ord16(C_ref))
    assert (d > 1).mean() < 0.01, (int(d.max()), float((d > 1).mean()))


def test_nf4_k_zero_gives_zeros(dev):
    from bit_mixed_precision_amd import bq
    import torch

    banner("nf4 K=0")
    A = torch.empty((5, 0), dtype=torch.float16, device=dev)
    B = torch.empty((7, 0), dtype=torch.uint8, device=dev)
    s = torch.ones(7, dtype=torch.float16, device=dev)
    C = bq.gemm_nf4_a16(A, B, s, out=torch.full((5, 7), 3.0, dtype=torch.float16, device=dev))
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0


@pytest.mark.parametrize("M", [4, 16])
def test_nf4_dequantized_weights_bit_exact(dev, M):
    """One-hot activation rows (A[m, k_m] = 1) make C[m, n] = W[n, k_m]
    exactly, so the GPU's dequantized weights -- fp16(fp32(table[c] - zero)
    * scale), two fp32 roundings then one to fp16 -- are compared bit for bit
    with the oracle's, for scales and zero points over a wide range
    (subnormal to 2^10), on the decode GEMV (M = 4) and the tiled kernel
    (up to the sign of zero: an exact sum of +0 and -0 terms is +0)."""
    N, K = 300, 256
    banner(f"nf4 dequantized weights M={M}")
    g = np.random.default_rng(M)
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    s = (g.choice([1, -1], N) * 2.0 ** g.integers(-24, 11, N) * (1 + g.integers(0, 1024, N) / 1024))
    z = (g.choice([1, -1], N) * 2.0 ** g.integers(-24, 4, N) * (1 + g.integers(0, 1024, N) / 1024))
    s = s.astype(np.float16).view(np.uint16)
    z = z.astype(np.float16).view(np.uint16)
    ks = g.choice(K, M, replace=False)
    A = np.zeros((M, K), np.float16)
    A[np.arange(M), ks] = 1.0
    Bp = nf4.pack_codes(codes)
    C = _run(dev, A.view(np.uint16), Bp, s, z)
    W = nf4.dequant_nf4(Bp, K, s, z)
    # a sum whose only nonzero term is -0 is +0
    want = np.where(W[:, ks].T == 0x8000, 0, W[:, ks].T).astype(np.uint16)
    bad = np.argwhere(C != want)
    assert len(bad) == 0, (f"{len(bad)} of {C.size} weights differ; first: " +
                           ", ".join(f"got {C[i, j]:#06x} want {want[i, j]:#06x}" for i, j in bad[:8]))
