"""GPU parity of the W8A8 / W4A8 / W2A8 GEMMs against the oracle, through the
C ABI.  int32 accumulators bit-exact; fp16 outputs within 1 ulp of the
correctly rounded acc*scale (the epilogue multiplies in fp32).

Small shapes span several tiles of both kernels with ragged M and N tails;
the workload shapes run in the launch configuration the benchmark uses
(automatic path selection) and are compared on sampled rows/columns that
the oracle computes one by one."""
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
    """Host inputs: A int8, B values, packed B (by the oracle), fp16 scale."""
    if bits == 8:
        A, Bv, s = synth.w8a8_case(M, N, K, seed)
        Bp = Bv
    elif bits == 4:
        A, Bv, s = synth.w4a8_case(M, N, K, seed)
        Bp = oracle.pack_int4(Bv)
    else:
        A, Bv, s = synth.w2a8_case(M, N, K, seed, ternary=(seed % 2 == 0))
        Bp = oracle.pack_int2(Bv)
    return A, Bv, Bp, s


def _run(dev, bits, A, Bp, s, path):
    from bit_mixed_precision_amd import bq
    import torch

    Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
    acc = bq.gemm(Ad, Bd, bits, None, path=path)
    C = bq.gemm(Ad, Bd, bits, sd, path=path)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), f16_bits(C)


def _check(acc, C, A, Bv, s, rows=None, cols=None, what=""):
    """Compare (optionally a sample of rows/cols of) the GPU results with the
    oracle computed on the same rows/cols."""
    rows = np.arange(A.shape[0]) if rows is None else rows
    cols = np.arange(Bv.shape[0]) if cols is None else cols
    acc_ref = oracle.gemm_i32(np.ascontiguousarray(A[rows]), np.ascontiguousarray(Bv[cols]))
    got = acc[np.ix_(rows, cols)]
    if not np.array_equal(got, acc_ref):
        bad = np.argwhere(got != acc_ref)
        i, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} int32 results differ; first at row "
                             f"{rows[i]} col {cols[j]}: got {got[i, j]} want {acc_ref[i, j]}")
    C_ref = oracle.dequant(acc_ref, s[cols])
    n1 = assert_f16_within_1ulp(C[np.ix_(rows, cols)], C_ref, what)
    return n1


SMALL = [(1, 16, 64), (1, 33, 128), (3, 100, 192), (16, 256, 256), (17, 48, 320),
         (33, 100, 320), (64, 520, 1024), (5, 4099, 128)]
# M up to 256 on the streaming and tiled paths; above 256 tiled only
MID = [(65, 300, 384), (130, 257, 256), (256, 513, 640), (200, 130, 64)]
TILED_ONLY = [(257, 513, 640), (300, 130, 64)]


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("path", ["gemv", "stream", "tiled"])
@pytest.mark.parametrize("shape", SMALL + [(2, 100, 64), (4, 37, 8192), (3, 4101, 640)])
def test_small_shapes_all_paths(dev, bits, path, shape):
    M, N, K = shape
    if path == "gemv" and M > 4:
        pytest.skip("the GEMV path takes M <= 4")
    banner(f"gemm bits={bits} path={path} M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=M + N + K + bits)
    acc, C = _run(dev, bits, A, Bp, s, path)
    _check(acc, C, A, Bv, s, what=f"w{bits} {path} {shape}")


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("path", ["stream", "tiled", "auto"])
@pytest.mark.parametrize("shape", MID)
def test_mid_shapes(dev, bits, path, shape):
    M, N, K = shape
    banner(f"gemm bits={bits} path={path} M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=M + N + K + bits)
    acc, C = _run(dev, bits, A, Bp, s, path)
    _check(acc, C, A, Bv, s, what=f"w{bits} {path} {shape}")


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("shape", TILED_ONLY)
def test_small_shapes_tiled(dev, bits, shape):
    M, N, K = shape
    banner(f"gemm bits={bits} path=auto(tiled) M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=M + N + K + bits)
    acc, C = _run(dev, bits, A, Bp, s, "auto")
    _check(acc, C, A, Bv, s, what=f"w{bits} auto {shape}")


# Shapes that select each tile configuration of the tiled path, with ragged
# M, N and K tails: 256x256 tiles (4100x4100), 128x128 (1030x4100), 64x64
# with a 4-stage ring (1000x2100, K tail of 64) and 64x64 with an 8-stage ring
# (the rest; 100x200x1088 has a K tail, 3x40x8192 a long K; none splits K:
# bq_gemm passes no workspace).
CFG_SHAPES = [(4100, 4100, 64), (1030, 4100, 128), (1000, 2100, 192), (200, 300, 1024),
              (100, 200, 1088), (3, 40, 8192), (130, 257, 256)]


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("shape", CFG_SHAPES)
def test_tile_configs(dev, bits, shape):
    M, N, K = shape
    banner(f"gemm bits={bits} path=tiled M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=M + N + K + bits)
    acc, C = _run(dev, bits, A, Bp, s, "tiled")
    _check(acc, C, A, Bv, s, what=f"w{bits} tiled {shape}")


def test_w4a8_16x256x256_full(dev):
    """The small W4A8 case: M=16, N=256, K=256, seed 0, compared in full."""
    banner("gemm w4a8 16x256x256 seed 0")
    A, Bv, s = synth.w4a8_case(16, 256, 256, seed=0)
    Bp = oracle.pack_int4(Bv)
    acc, C = _run(dev, 4, A, Bp, s, "auto")
    _check(acc, C, A, Bv, s, what="w4a8 16x256x256")


@pytest.mark.parametrize("N", [4096, 11008])
def test_decode_gemv_w4a8_full(dev, N):
    banner(f"gemm w4a8 decode M=1 N={N} K=4096")
    A, Bv, s = synth.w4a8_case(1, N, 4096, seed=0)
    acc, C = _run(dev, 4, A, oracle.pack_int4(Bv), s, "auto")
    _check(acc, C, A, Bv, s, what=f"w4a8 1x{N}x4096")


@pytest.mark.parametrize("M", [1, 128])
def test_ternary_w2a8_workload(dev, M):
    """The ternary W2A8 workload at M = 1 and 128, N = K = 4096, every output
    compared."""
    banner(f"gemm w2a8 ternary M={M} N=4096 K=4096")
    A, Bv, s = synth.w2a8_case(M, 4096, 4096, seed=0)
    acc, C = _run(dev, 2, A, oracle.pack_int2(Bv), s, "auto")
    _check(acc, C, A, Bv, s, what=f"w2a8 {M}x4096x4096")


def test_bminf_quantize_then_w8a8(dev):
    """Quantized fused-QKV weight [12288, 4096] (codes and scales from the
    oracle) times int8 activations, M=64, every output compared."""
    banner("gemm w8a8 bminf M=64 N=12288 K=4096")
    W, A = synth.bminf_case()
    q, s = oracle.quantize_rows(W)
    acc, C = _run(dev, 8, A, q, s.view(np.float16), "auto")
    _check(acc, C, A, q, s.view(np.float16), what="w8a8 bminf")


@pytest.mark.parametrize("M", [1, 16, 64, 256, 1024, 4096])
def test_w4a8_prefill_sweep(dev, M):
    """The W4A8 sweep, N = K = 4096, every output compared (the M = 4096
    oracle is one 4096^3 integer GEMM on the host cores, about 2 s)."""
    banner(f"gemm w4a8 sweep M={M} N=4096 K=4096")
    A, Bv, s = synth.w4a8_case(M, 4096, 4096, seed=0)
    acc, C = _run(dev, 4, A, oracle.pack_int4(Bv), s, "auto")
    _check(acc, C, A, Bv, s, what=f"w4a8 sweep M={M}")


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 1024), (4100, 4130, 576)])
def test_largest_tile_configuration(dev, bits, M, N, K):
    """The 256 x 256 tile configuration (chosen once there are 256 such tiles)
    for every weight width, int32 and fp16 outputs, without and with M, N and
    K tails (K = 576 ends in half a 128-k stage); sampled rows and columns,
    the ragged last tile row and column included."""
    banner(f"gemm largest tiles w{bits} M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(bits, M, N, K, seed=M + N + K + bits)
    acc, C = _run(dev, bits, A, Bp, s, "auto")
    g = np.random.default_rng(M + N + bits)
    rows = np.unique(np.concatenate([g.choice(M, 64, replace=False), np.arange(M - 8, M), [0]]))
    cols = np.unique(np.concatenate([g.choice(N, 768, replace=False), np.arange(N - 40, N), [0]]))
    _check(acc, C, A, Bv, s, rows=rows, cols=cols, what=f"w{bits} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 8192), (4352, 4160, 4160)])
def test_pingpong_loop_int4(dev, M, N, K):
    """The 256 x 256 int4 tiles' ping-pong K loop: 64 stages, and 33 stages
    ending in half a stage (K = 4160) with ragged last tile rows and
    columns (17 x 17 tiles); int32 and fp16 outputs on sampled rows and
    columns, the last ones included."""
    banner(f"gemm pingpong int4 M={M} N={N} K={K}")
    A, Bv, Bp, s = _make(4, M, N, K, seed=M + N + K)
    acc, C = _run(dev, 4, A, Bp, s, "auto")
    g = np.random.default_rng(K)
    rows = np.unique(np.concatenate([g.choice(M, 48, replace=False), np.arange(M - 4, M), [0, 255, 256]]))
    cols = np.unique(np.concatenate([g.choice(N, 512, replace=False), np.arange(N - 70, N), [0, 255, 256]]))
    _check(acc, C, A, Bv, s, rows=rows, cols=cols, what=f"w4 pingpong {M}x{N}x{K}")


@pytest.mark.parametrize("K", [0, 64, 128, 256, 384])
def test_pingpong_short_k(dev, K):
    """The ping-pong loop with 0-3 stages of K (K = 64: one stage, half of it
    past K), where its prologue's and last steps' loads past the end and its
    group barriers meet: every column of 288 rows (each tile's first and last
    rows among them), int32 and fp16, against the oracle; K = 0 gives zeros
    everywhere."""
    from bit_mixed_precision_amd import bq
    import torch

    M = N = 4096
    banner(f"gemm pingpong short K={K}")
    if K == 0:
        A = torch.zeros((M, 0), dtype=torch.int8, device=dev)
        B = torch.zeros((N, 0), dtype=torch.uint8, device=dev)
        s = torch.ones((N,), dtype=torch.float16, device=dev)
        C = bq.gemm(A, B, 4, s, out=torch.full((M, N), 7.0, dtype=torch.float16, device=dev))
        acc = bq.gemm(A, B, 4, None, out=torch.full((M, N), 7, dtype=torch.int32, device=dev))
        torch.cuda.synchronize()
        assert not acc.cpu().numpy().any()
        assert not f16_bits(C).any()
        return
    A, Bv, Bp, s = _make(4, M, N, K, seed=K + 11)
    acc, C = _run(dev, 4, A, Bp, s, "auto")
    g = np.random.default_rng(K)
    rows = np.unique(np.concatenate([g.choice(M, 256, replace=False), np.arange(0, M, 256), np.arange(255, M, 256)]))
    _check(acc, C, A, Bv, s, rows=rows, what=f"w4 pingpong short K={K}")


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("path", ["gemv", "stream", "tiled"])
def test_k_zero_and_empty(dev, bits, path):
    from bit_mixed_precision_amd import bq
    import torch

    banner(f"gemm K=0 / empty bits={bits} path={path}")
    A = torch.zeros((3, 0), dtype=torch.int8, device=dev)
    B = torch.zeros((5, 0), dtype=torch.int8 if bits == 8 else torch.uint8, device=dev)
    s = torch.ones((5,), dtype=torch.float16, device=dev)
    C = bq.gemm(A, B, bits, s, out=torch.full((3, 5), 7.0, dtype=torch.float16, device=dev), path=path)
    acc = bq.gemm(A, B, bits, None, out=torch.full((3, 5), 7, dtype=torch.int32, device=dev), path=path)
    torch.cuda.synchronize()
    assert not acc.cpu().numpy().any()
    assert not f16_bits(C).any()
    # M = 0 and N = 0 are no-ops
    bq.gemm(torch.zeros((0, 64), dtype=torch.int8, device=dev),
            torch.zeros((5, 64 * bits // 8), dtype=B.dtype, device=dev), bits, s, path=path)
    torch.cuda.synchronize()


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("path", ["gemv", "stream", "tiled"])
def test_max_k_extremes(dev, bits, path):
    """K = 65536 (the largest accepted) with the largest-magnitude operands."""
    banner(f"gemm K=65536 extremes bits={bits} path={path}")
    K = 65536
    M, N = 3, 40
    A = np.full((M, K), -128, np.int8)
    A[1] = 127
    A[2, ::2] = -128
    A[2, 1::2] = 127
    vmin = {8: -128, 4: -8, 2: -2}[bits]
    vmax = {8: 127, 4: 7, 2: 1}[bits]
    Bv = np.full((N, K), vmin, np.int8)
    Bv[1::2] = vmax
    Bv[5, :K // 2] = 0
    Bp = Bv if bits == 8 else (oracle.pack_int4(Bv) if bits == 4 else oracle.pack_int2(Bv))
    s = np.full(N, 2.0 ** -24, np.float16)
    s[::3] = 2.0 ** -14
    acc, C = _run(dev, bits, A, Bp, s, path)
    _check(acc, C, A, Bv, s, what=f"K max w{bits} {path}")


def test_named_entry_points_agree(dev):
    """The six named calls give the results of the general call."""
    from bit_mixed_precision_amd import bq
    import torch

    banner("named entry points")
    for bits in (8, 4, 2):
        for M in (7, 100):
            A, Bv, Bp, s = _make(bits, M, 200, 256, seed=bits + M)
            Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
            acc = getattr(bq, f"gemm_w{bits}a8_i32")(Ad, Bd)
            C = getattr(bq, f"gemm_w{bits}a8_dequant")(Ad, Bd, sd)
            torch.cuda.synchronize()
            _check(acc.cpu().numpy(), f16_bits(C), A, Bv, s, what=f"named w{bits} M={M}")


def test_error_paths(dev):
    from bit_mixed_precision_amd import bq
    import torch

    banner("error paths")
    A = torch.zeros((4, 96), dtype=torch.int8, device=dev)
    B = torch.zeros((4, 96), dtype=torch.int8, device=dev)
    with pytest.raises(bq.BQError) as e:
        bq.gemm(A, B, 8)  # K % 64 != 0
    assert e.value.status == bq.BQ_ERR_SHAPE
    buf = torch.zeros((4 * 64 + 1,), dtype=torch.int8, device=dev)
    Au = buf[1:].view(4, 64)  # misaligned by one byte
    with pytest.raises(bq.BQError) as e:
        bq.gemm(Au, torch.zeros((4, 64), dtype=torch.int8, device=dev), 8)
    assert e.value.status == bq.BQ_ERR_ALIGN
    with pytest.raises(bq.BQError) as e:
        bq.gemm(torch.zeros((257, 64), dtype=torch.int8, device=dev),
                torch.zeros((4, 64), dtype=torch.int8, device=dev), 8, path="stream")
    assert e.value.status == bq.BQ_ERR_SHAPE
    with pytest.raises(bq.BQError) as e:
        bq.gemm(torch.zeros((5, 64), dtype=torch.int8, device=dev),
                torch.zeros((4, 64), dtype=torch.int8, device=dev), 8, path="gemv")
    assert e.value.status == bq.BQ_ERR_SHAPE


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("N", [6143, 6144, 6145, 6200])
def test_decode_gemv_rows_rule_boundary(dev, bits, M, N):
    """Around the 6144-rows-per-launch switch between wavefront shapes (one or
    two B rows per wavefront, four to sixteen wavefronts per workgroup, by
    bits and M; ragged last workgroup with idle wavefronts), K = 1024,
    compared in full."""
    banner(f"gemm decode rows-rule boundary bits={bits} M={M} N={N}")
    A, Bv, Bp, s = _make(bits, M, N, 1024, seed=N + bits + 7 * M)
    acc, C = _run(dev, bits, A, Bp, s, "gemv")
    _check(acc, C, A, Bv, s, what=f"w{bits} gemv {M}x{N}x1024")


@pytest.mark.parametrize("bits", [4, 2])
def test_decode_gemv_batched_rows_rule(dev, bits):
    """Batched M = 1 GEMV where N x batch crosses the 6144-row switch
    (3 x 2112 = 6336 rows and 2 x 2112 fall on either side of it; 2112 keeps
    every batch's scale and output 16-byte aligned)."""
    import torch

    from bit_mixed_precision_amd import bq

    for batch in (2, 3):
        banner(f"gemm decode batched rows rule bits={bits} batch={batch}")
        A, Bv, Bp, s = _make(bits, 1, 2112 * batch, 512, seed=batch * 10 + bits)
        Bb = to_dev(Bp.reshape(batch, 2112, -1), dev)
        sb = to_dev(s.reshape(batch, 2112), dev)
        C = bq.gemm_batched(to_dev(A, dev), Bb, bits, sb, path="gemv")
        acc = bq.gemm_batched(to_dev(A, dev), Bb, bits, None, path="gemv")
        torch.cuda.synchronize()
        got_acc = acc.cpu().numpy().transpose(1, 0, 2).reshape(1, -1)
        got_C = f16_bits(C).transpose(1, 0, 2).reshape(1, -1)
        _check(got_acc, got_C, A, Bv, s, what=f"w{bits} batched gemv x{batch}")
