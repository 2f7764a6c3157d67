"""Pins for the oracle's integer GEMM (BitBLAS guide, section 1:
C[i,j] = sum_k int32(A[i,k]) * int32(B[j,k]), B stored [N, K]) and dequant
epilogue (section 2: the int32 result times scale[j], as fp16).

Independent checks: a pure-Python triple loop on tiny shapes, numpy's exact
int64 matmul, the blocked-K identity of the Pallas page's block matmul
(a sum of per-block partial products over K equals the full product,
checked there with an exact array comparison), and numpy's / Fraction's
rounding of the exact product for the epilogue.
"""
from fractions import Fraction

import numpy as np
import pytest

from bit_mixed_precision_amd import synth


def _triple_loop(A, B):
    M, K = A.shape
    N = B.shape[0]
    C = [[0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0
            for k in range(K):
                s += int(A[i, k]) * int(B[j, k])
            C[i][j] = s
    return np.array(C, np.int64)


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (8, 8, 16), (4, 9, 13)])
def test_triple_loop(oracle, shape):
    M, N, K = shape
    g = np.random.default_rng(sum(shape))
    A = g.integers(-128, 128, (M, K), dtype=np.int8)
    B = g.integers(-128, 128, (N, K), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i32(A, B), _triple_loop(A, B))


def test_sign_combinations(oracle):
    ext = np.array([-128, -127, -1, 0, 1, 127], np.int8)
    A = np.array(np.meshgrid(ext, ext)).reshape(2, -1).T.astype(np.int8)  # 36 x 2
    B = A.copy()
    assert np.array_equal(oracle.gemm_i32(A, B), _triple_loop(A, B))


def test_numpy_int64_matmul_and_packed(oracle):
    A, B4, _ = synth.w4a8_case(37, 70, 384, seed=1)
    ref = A.astype(np.int64) @ B4.astype(np.int64).T
    assert np.array_equal(oracle.gemm_i32(A, B4), ref)
    assert np.array_equal(oracle.gemm_wxa8_i32(A, oracle.pack_int4(B4), 4), ref)
    _, B2, _ = synth.w2a8_case(37, 70, 384, seed=2, ternary=False)
    ref2 = A.astype(np.int64) @ B2.astype(np.int64).T
    assert np.array_equal(oracle.gemm_wxa8_i32(A, oracle.pack_int2(B2), 2), ref2)


@pytest.mark.parametrize("bk", [1, 64, 256, 512])
def test_blocked_k_identity(oracle, bk):
    A, B, _ = synth.w8a8_case(16, 24, 512, seed=5)
    full = oracle.gemm_i32(A, B).astype(np.int64)
    acc = np.zeros_like(full)
    for k0 in range(0, 512, bk):
        acc += oracle.gemm_i32(np.ascontiguousarray(A[:, k0:k0 + bk]),
                               np.ascontiguousarray(B[:, k0:k0 + bk]))
    assert np.array_equal(acc, full)


def test_int32_range(oracle):
    K = 65536
    A = np.full((1, K), -128, np.int8)
    B = np.full((1, K), -128, np.int8)
    assert int(oracle.gemm_i32(A, B)[0, 0]) == 2 ** 30
    K = 131072  # 2^31 does not fit in int32: the oracle refuses
    with pytest.raises(oracle.OracleError):
        oracle.gemm_i32(np.full((1, K), -128, np.int8), np.full((1, K), -128, np.int8))


def test_empty_shapes(oracle):
    assert oracle.gemm_i32(np.zeros((0, 4), np.int8), np.zeros((3, 4), np.int8)).shape == (0, 3)
    C = oracle.gemm_i32(np.zeros((2, 0), np.int8), np.zeros((3, 0), np.int8))
    assert C.shape == (2, 3) and not C.any()


def test_dequant_matches_numpy_rounding(oracle):
    g = np.random.default_rng(11)
    acc = g.integers(-2_000_000, 2_000_000, (64, 96), dtype=np.int32)
    acc[0, :10] = [0, 1, -1, 2**31 - 1, -2**31, 65504, 65519, 65520, 2049, 2051]
    s = synth.fp16_uniform(g, 96, 0.0005, 0.02)
    s[:10] = 1.0
    with np.errstate(over="ignore"):
        ref = (acc.astype(np.float64) * s.astype(np.float64)[None, :]).astype(np.float16)
    got = oracle.dequant(acc, s)
    assert np.array_equal(got, ref.view(np.uint16))
    # ties to even at the fp16 grid spacing of 2 in [2048, 4096)
    assert got[0, 8] == np.float16(2048).view(np.uint16)
    assert got[0, 9] == np.float16(2052).view(np.uint16)
    assert got[0, 6] == np.float16(65504).view(np.uint16)
    assert got[0, 7] == 0x7C00 and got[0, 0] == 0


def test_dequant_exact_fraction_sample(oracle):
    g = np.random.default_rng(12)
    acc = g.integers(-90_000, 90_000, (4, 64), dtype=np.int32)
    s = synth.fp16_uniform(g, 64, 0.001, 0.01)
    got = oracle.dequant(acc, s).view(np.float16)
    for i in range(4):
        for j in range(64):
            exact = Fraction(int(acc[i, j])) * Fraction(float(s[j]))
            v = Fraction(float(got[i, j]))
            # nearest: no other fp16 is strictly closer; ties resolved to even
            bits = int(got[i:i + 1, j].view(np.uint16)[0])
            for nb in (bits - 1, bits + 1):
                w = Fraction(float(np.uint16(nb).view(np.float16)))
                assert abs(w - exact) > abs(v - exact) or (
                    abs(w - exact) == abs(v - exact) and bits % 2 == 0)
