"""The C ABI library loads, exports every entry point declared in
include/bq.h, and rejects invalid arguments on the host before any device
call (no compute call is made here; these tests run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bq.h")


@pytest.fixture(scope="module")
def bq():
    from bit_mixed_precision_amd import bq as _bq

    if not os.path.exists(_bq.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return _bq


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(bq):
    names = _declared()
    assert len(names) == 22, names
    lib = ctypes.CDLL(bq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bq.SIGNATURES)


def test_version_and_status_strings(bq):
    assert bq.version() == 100
    for st in range(7):
        assert bq.status_string(st)
    assert bq.status_string(0) == "ok"
    assert "unknown" in bq.status_string(99)


def test_select_path(bq):
    assert bq.select_path(1, 4096, 4096, 4) == "gemv"
    assert bq.select_path(2, 4096, 4096, 2) == "gemv"
    assert bq.select_path(3, 4096, 4096, 4) == "stream"
    assert bq.select_path(64, 4096, 4096, 4) == "stream"
    assert bq.select_path(64, 12288, 4096, 8) == "stream"
    assert bq.select_path(128, 4096, 4096, 2) == "stream"
    assert bq.select_path(129, 4096, 4096, 4) == "tiled"
    assert bq.select_path(256, 4096, 4096, 2) == "stream"
    assert bq.select_path(257, 4096, 4096, 2) == "tiled"
    assert bq.select_path(4096, 4096, 4096, 2) == "tiled"


# Fake, never-dereferenced device addresses: validation fails before any
# HIP call, so nothing touches them.
P16 = ctypes.c_void_p(0x1000)
P16b = ctypes.c_void_p(0x2000)
P16c = ctypes.c_void_p(0x3000)
P16d = ctypes.c_void_p(0x4000)
PODD = ctypes.c_void_p(0x1001)
NULL = ctypes.c_void_p(0)


def test_gemm_validation(bq):
    L = bq.lib()
    S = NULL  # stream
    # bad bits / path
    assert L.bq_gemm(P16, P16b, 3, P16c, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ARG
    assert L.bq_gemm(P16, P16b, 4, P16c, P16d, 4, 4, 64, 7, S) == bq.BQ_ERR_ARG
    # shapes
    for M, N, K in [(-1, 4, 64), (4, -1, 64), (4, 4, -64), (4, 4, 32), (4, 4, 100),
                    (4, 4, 65536 + 64), (2**31, 4, 64), (2**30 + 1, 4, 64), (4, 2**30 + 1, 64),
                    (2**30, 2**12 + 1, 64), (2**21, 2**21 + 1, 64)]:
        assert L.bq_gemm(P16, P16b, 8, P16c, P16d, M, N, K, 0, S) == bq.BQ_ERR_SHAPE, (M, N, K)
    # the dimension and output limits are inclusive: the next check (NULL) decides
    assert L.bq_gemm(NULL, P16b, 8, P16c, P16d, 2**30, 4, 64, 0, S) == bq.BQ_ERR_NULL
    assert L.bq_gemm(NULL, P16b, 8, P16c, P16d, 2**21, 2**21, 64, 0, S) == bq.BQ_ERR_NULL
    # the streaming kernel only takes M <= 256
    assert L.bq_gemm(P16, P16b, 8, P16c, P16d, 257, 4, 64, 1, S) == bq.BQ_ERR_SHAPE
    # the GEMV path only takes M <= 4
    assert L.bq_gemm(P16, P16b, 8, P16c, P16d, 5, 4, 64, 3, S) == bq.BQ_ERR_SHAPE
    # nulls
    assert L.bq_gemm(NULL, P16b, 8, P16c, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_NULL
    assert L.bq_gemm(P16, NULL, 8, P16c, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_NULL
    assert L.bq_gemm(P16, P16b, 8, P16c, NULL, 4, 4, 64, 0, S) == bq.BQ_ERR_NULL
    assert L.bq_gemm_w4a8_dequant(P16, P16b, NULL, P16d, 4, 4, 64, S) == bq.BQ_ERR_NULL
    # alignment
    assert L.bq_gemm(PODD, P16b, 8, P16c, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm(P16, PODD, 8, P16c, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm(P16, P16b, 8, PODD, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm(P16, P16b, 8, P16c, PODD, 4, 4, 64, 0, S) == bq.BQ_ERR_ALIGN
    # empty outputs are valid no-ops (no device call needed)
    assert L.bq_gemm(NULL, NULL, 8, NULL, NULL, 0, 4, 64, 0, S) == bq.BQ_OK
    assert L.bq_gemm(NULL, NULL, 4, NULL, NULL, 4, 0, 64, 0, S) == bq.BQ_OK
    assert L.bq_gemm_w2a8_i32(NULL, NULL, NULL, 0, 0, 0, S) == bq.BQ_OK


def test_splitk_workspace_bytes(bq):
    """The workspace size follows the header's contract: 0 where K is not
    split (more than 128 output tiles of 64 x 64, or K below 1024), else
    4096 counter bytes plus 16 KiB per workgroup, at most 256 workgroups."""
    f = bq.gemm_splitk_workspace_bytes
    assert f(4096, 4096, 4096, 4) == 0          # 4096 tiles
    assert f(64, 64 * 129, 4096, 8) == 0        # 129 tiles
    assert f(64, 4096, 512, 4) == 0             # K too short to split
    cap = 4096 + 256 * 16384
    for bits in (8, 4, 2):
        for M, N, K in [(64, 4096, 4096), (3, 40, 8192), (128, 512, 4160), (200, 300, 8192)]:
            n = f(M, N, K, bits)
            tiles = -(-M // 64) * -(-N // 64)
            assert n > 4096 and (n - 4096) % 16384 == 0, (M, N, K, n)
            wgs = (n - 4096) // 16384
            assert wgs % tiles == 0 and 2 <= wgs // tiles <= 8 and wgs <= 256, (M, N, K, wgs)
            assert n <= cap
    assert f(0, 4096, 4096, 4) == 0
    with pytest.raises(bq.BQError):
        f(64, 64, 96, 4)
    with pytest.raises(bq.BQError):
        f(64, 64, 4096, 3)


def test_splitk_validation(bq):
    L = bq.lib()
    S = NULL
    f = L.bq_gemm_splitk
    assert f(P16, P16b, 4, P16c, P16d, 64, 64, 4096, P16, -1, S) == bq.BQ_ERR_SHAPE
    assert f(P16, P16b, 4, P16c, P16d, 64, 64, 4096, NULL, 4096, S) == bq.BQ_ERR_NULL
    assert f(P16, P16b, 4, P16c, P16d, 64, 64, 4096, PODD, 4096, S) == bq.BQ_ERR_ALIGN
    # the shared checks of bq_gemm apply
    assert f(P16, P16b, 3, P16c, P16d, 64, 64, 4096, P16, 4096, S) == bq.BQ_ERR_ARG
    assert f(P16, P16b, 4, P16c, P16d, 64, 64, 96, P16, 4096, S) == bq.BQ_ERR_SHAPE
    assert f(NULL, NULL, 4, NULL, NULL, 0, 64, 4096, NULL, 0, S) == bq.BQ_OK


def test_splitk_static_validation(bq):
    """The allocation-free entry point validates like bq_gemm before any
    device call."""
    L = bq.lib()
    S = NULL
    f = L.bq_gemm_splitk_static
    assert f(P16, P16b, 3, P16c, P16d, 64, 64, 4096, S) == bq.BQ_ERR_ARG
    assert f(P16, P16b, 4, P16c, P16d, 64, 64, 96, S) == bq.BQ_ERR_SHAPE
    assert f(P16, P16b, 4, P16c, P16d, 64, 64, 65536 + 64, S) == bq.BQ_ERR_SHAPE
    assert f(NULL, P16b, 4, P16c, P16d, 64, 64, 4096, S) == bq.BQ_ERR_NULL
    assert f(PODD, P16b, 4, P16c, P16d, 64, 64, 4096, S) == bq.BQ_ERR_ALIGN
    assert f(NULL, NULL, 4, NULL, NULL, 0, 64, 4096, S) == bq.BQ_OK
    # every shape's split fits the static scratch (4 MiB + 4 KiB)
    cap = 4096 + 256 * 16384
    for M, N, K in [(64, 4096, 4096), (3, 40, 65536), (128, 8192, 65536), (1, 64 * 128, 65536)]:
        assert bq.gemm_splitk_workspace_bytes(M, N, K, 8) <= cap


def test_quantize_bits_validation(bq):
    L = bq.lib()
    S = NULL
    for bits in (0, 1, 3, 16):
        assert L.bq_quantize_rows_bits(P16, 4, 64, bits, P16b, P16c, S) == bq.BQ_ERR_ARG
    assert L.bq_quantize_rows_bits(P16, -1, 64, 4, P16b, P16c, S) == bq.BQ_ERR_SHAPE
    assert L.bq_quantize_rows_bits(P16, 4, 64, 4, P16b, NULL, S) == bq.BQ_ERR_NULL
    assert L.bq_quantize_rows_bits(PODD, 4, 64, 4, P16b, P16c, S) == bq.BQ_ERR_ALIGN
    assert L.bq_quantize_rows_bits(NULL, 0, 64, 2, NULL, NULL, S) == bq.BQ_OK


def test_quantize_pack_validation(bq):
    L = bq.lib()
    S = NULL
    for bits in (0, 1, 3, 8):
        assert L.bq_quantize_pack(P16, 4, 64, bits, P16b, P16c, S) == bq.BQ_ERR_ARG
    assert L.bq_quantize_pack(P16, -1, 64, 4, P16b, P16c, S) == bq.BQ_ERR_SHAPE
    assert L.bq_quantize_pack(P16, 4, 63, 4, P16b, P16c, S) == bq.BQ_ERR_SHAPE
    assert L.bq_quantize_pack(P16, 4, 66, 2, P16b, P16c, S) == bq.BQ_ERR_SHAPE
    assert L.bq_quantize_pack(P16, 4, 64, 4, P16b, NULL, S) == bq.BQ_ERR_NULL
    assert L.bq_quantize_pack(P16, 4, 64, 2, NULL, P16c, S) == bq.BQ_ERR_NULL
    assert L.bq_quantize_pack(PODD, 4, 64, 4, P16b, P16c, S) == bq.BQ_ERR_ALIGN
    assert L.bq_quantize_pack(NULL, 0, 64, 2, NULL, NULL, S) == bq.BQ_OK


def test_act_validation(bq):
    L = bq.lib()
    S = NULL
    assert L.bq_gemm_act(P16, P16b, 8, P16c, NULL, 3, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ARG
    assert L.bq_gemm_act(P16, P16b, 8, P16c, NULL, -1, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ARG
    assert L.bq_gemm_act(P16, P16b, 8, NULL, NULL, 2, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_NULL
    assert L.bq_gemm_act(P16, P16b, 8, P16c, PODD, 2, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm_act(P16, P16b, 8, P16c, NULL, 1, P16d, 4, 4, 96, 0, S) == bq.BQ_ERR_SHAPE
    assert L.bq_gemm_act(NULL, NULL, 8, NULL, NULL, 2, NULL, 0, 4, 64, 0, S) == bq.BQ_OK


def test_dual_scale_validation(bq):
    L = bq.lib()
    S = NULL
    # both scales are required; the token scale must be aligned
    assert L.bq_gemm_dual_scale(P16, P16b, 8, NULL, P16c, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_NULL
    assert L.bq_gemm_dual_scale(P16, P16b, 8, P16c, NULL, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_NULL
    assert L.bq_gemm_dual_scale(P16, P16b, 8, P16c, PODD, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ALIGN
    # the shared checks of bq_gemm apply
    assert L.bq_gemm_dual_scale(P16, P16b, 3, P16c, P16c, P16d, 4, 4, 64, 0, S) == bq.BQ_ERR_ARG
    assert L.bq_gemm_dual_scale(P16, P16b, 8, P16c, P16c, P16d, 4, 4, 96, 0, S) == bq.BQ_ERR_SHAPE
    assert L.bq_gemm_dual_scale(P16, P16b, 8, P16c, P16c, PODD, 4, 4, 64, 0, S) == bq.BQ_ERR_ALIGN
    assert L.bq_gemm_dual_scale(NULL, NULL, 8, NULL, NULL, NULL, 0, 4, 64, 0, S) == bq.BQ_OK


def test_quantize_and_pack_validation(bq):
    L = bq.lib()
    S = NULL
    assert L.bq_quantize_rows(P16, -1, 8, P16b, P16c, S) == bq.BQ_ERR_SHAPE
    assert L.bq_quantize_rows(P16, 4, -8, P16b, P16c, S) == bq.BQ_ERR_SHAPE
    assert L.bq_quantize_rows(NULL, 4, 8, P16b, P16c, S) == bq.BQ_ERR_NULL
    assert L.bq_quantize_rows(P16, 4, 8, P16b, NULL, S) == bq.BQ_ERR_NULL
    assert L.bq_quantize_rows(PODD, 4, 8, P16b, P16c, S) == bq.BQ_ERR_ALIGN
    assert L.bq_quantize_rows(NULL, 0, 8, NULL, NULL, S) == bq.BQ_OK
    assert L.bq_pack_int4(P16, 4, 3, P16b, S) == bq.BQ_ERR_SHAPE
    assert L.bq_pack_int2(P16, 4, 6, P16b, S) == bq.BQ_ERR_SHAPE
    assert L.bq_pack_int4(P16, -4, 8, P16b, S) == bq.BQ_ERR_SHAPE
    assert L.bq_pack_int4(NULL, 4, 8, P16b, S) == bq.BQ_ERR_NULL
    assert L.bq_pack_int2(P16, 4, 8, PODD, S) == bq.BQ_ERR_ALIGN
    assert L.bq_pack_int4(NULL, 0, 8, NULL, S) == bq.BQ_OK
    assert L.bq_pack_int2(NULL, 4, 0, NULL, S) == bq.BQ_OK


def test_nf4_validation(bq):
    L = bq.lib()
    S = NULL
    f = L.bq_gemm_nf4_a16
    assert f(P16, P16b, P16c, NULL, P16d, 4, 4, 96, S) == bq.BQ_ERR_SHAPE   # K % 64
    assert f(P16, P16b, P16c, NULL, P16d, -1, 4, 64, S) == bq.BQ_ERR_SHAPE
    assert f(P16, P16b, P16c, NULL, P16d, 4, 4, 65536 + 64, S) == bq.BQ_ERR_SHAPE
    assert f(P16, P16b, P16c, NULL, P16d, 2**30 + 1, 4, 64, S) == bq.BQ_ERR_SHAPE
    assert f(P16, P16b, P16c, NULL, P16d, 2**21, 2**21 + 1, 64, S) == bq.BQ_ERR_SHAPE
    assert f(NULL, P16b, P16c, NULL, P16d, 2**21, 2**21, 64, S) == bq.BQ_ERR_NULL
    assert f(P16, P16b, NULL, NULL, P16d, 4, 4, 64, S) == bq.BQ_ERR_NULL    # scale required
    assert f(NULL, P16b, P16c, NULL, P16d, 4, 4, 64, S) == bq.BQ_ERR_NULL
    assert f(P16, P16b, P16c, PODD, P16d, 4, 4, 64, S) == bq.BQ_ERR_ALIGN   # zero point
    assert f(P16, PODD, P16c, NULL, P16d, 4, 4, 64, S) == bq.BQ_ERR_ALIGN
    assert f(NULL, NULL, NULL, NULL, NULL, 0, 4, 64, S) == bq.BQ_OK
    assert f(NULL, NULL, NULL, NULL, NULL, 4, 0, 64, S) == bq.BQ_OK


def test_calib_library_exports(bq):
    """The benchmark's measurement kernels (libbq_calib.so) load and export
    their two entry points; argument checks run on the host."""
    from bit_mixed_precision_amd import _build

    if not os.path.exists(_build.CALIB_LIB):
        _build.build_calib()
    lib = ctypes.CDLL(_build.CALIB_LIB)
    for name in ("bq_calib_mfma_loop", "bq_calib_mfma_w4a8_stream", "bq_calib_read_stream"):
        assert hasattr(lib, name), name
    # invalid arguments are rejected before any launch (no GPU needed)
    assert lib.bq_calib_mfma_loop(0, 1, None, None) != 0
    assert lib.bq_calib_mfma_w4a8_stream(0, 1, None, None) != 0
    assert lib.bq_calib_read_stream(None, ctypes.c_int64(16), 1, None, None) != 0
