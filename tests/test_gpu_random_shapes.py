"""GPU parity on seeded random shapes: every GEMM path against the oracle.

The fixed shape lists of the other GEMM tests are chosen to hit each tile
configuration and tail; this sweep draws M, N and K at random (seeded), so
that tails of every size meet every configuration and the staged int32 /
fp16 epilogues.  int32 accumulators must match bit for bit,
fp16 outputs within one fp16 ulp of the correctly rounded acc * scale."""
import numpy as np
import pytest

import oracle
from bit_mixed_precision_amd import synth
from gpu_util import assert_f16_within_1ulp, banner, f16_bits, need_gpu, to_dev

pytestmark = pytest.mark.gpu


def _cases(n=30, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        bits = (8, 4, 2)[i % 3]
        M = int(np.exp(g.uniform(0.0, np.log(600))))
        N = int(g.integers(1, 900))
        K = 64 * int(g.integers(1, 48))
        paths = ["auto", "tiled"] + (["stream"] if M <= 256 else []) + (["gemv"] if M <= 4 else [])
        out.append((bits, max(M, 1), N, K, paths[int(g.integers(0, len(paths)))], int(g.integers(0, 1 << 30))))
    # large outputs with short K, so that the 128 x 128 and 256 x 256 tile
    # configurations meet random tails too
    for i in range(6):
        bits = (8, 4, 2)[i % 3]
        if i < 4:
            M, N = int(g.integers(700, 1400)), int(g.integers(2100, 4300))
        else:
            M, N = int(g.integers(3900, 4300)), int(g.integers(3900, 4300))
        K = 64 * int(g.integers(1, 5))
        out.append((bits, M, N, K, "tiled", int(g.integers(0, 1 << 30))))
    return out


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


@pytest.mark.parametrize("bits,M,N,K,path,seed", _cases())
def test_random_shape_parity(dev, bits, M, N, K, path, seed):
    import torch

    from bit_mixed_precision_amd import bq

    banner(f"gemm random bits={bits} M={M} N={N} K={K} path={path} seed={seed}")
    if bits == 8:
        A, Bv, s = synth.w8a8_case(M, N, K, seed)
        Bp = Bv
    elif bits == 4:
        A, Bv, s = synth.w4a8_case(M, N, K, seed)
        Bp = oracle.pack_int4(Bv)
    else:
        A, Bv, s = synth.w2a8_case(M, N, K, seed, ternary=(seed % 2 == 0))
        Bp = oracle.pack_int2(Bv)
    Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
    acc = bq.gemm(Ad, Bd, bits, None, path=path)
    C = bq.gemm(Ad, Bd, bits, sd, path=path)
    torch.cuda.synchronize()
    acc_ref = oracle.gemm_i32(A, Bv)
    got = acc.cpu().numpy()
    if not np.array_equal(got, acc_ref):
        bad = np.argwhere(got != acc_ref)
        i, j = bad[0]
        raise AssertionError(f"{len(bad)} int32 results differ; first at ({i}, {j}): "
                             f"got {got[i, j]} want {acc_ref[i, j]}")
    assert_f16_within_1ulp(f16_bits(C), oracle.dequant(acc_ref, s), f"w{bits} {path} {M}x{N}x{K}")
