"""The allocation-free split-K entry point, bq_gemm_splitk_static (scratch in
a static device array of the library), against the entry point it varies,
bq_gemm_splitk (caller workspace), through the C ABI: two calls in a row,
the second with a smaller input (64 tiles x 4 parts of K, then 1 tile x 8),
each equal bit for bit to the workspace call and exact against the oracle;
and the device's free memory is unchanged by the calls."""
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


def _make(bits, M, N, K, seed):
    if bits == 4:
        A, Bv, s = synth.w4a8_case(M, N, K, seed)
        return A, Bv, oracle.pack_int4(Bv), s
    A, Bv, s = synth.w2a8_case(M, N, K, seed, ternary=True)
    return A, Bv, oracle.pack_int2(Bv), s


def test_static_scratch_matches_workspace_call(dev):
    import torch

    from bit_mixed_precision_amd import bq

    L = bq.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(0 if t is None else t.data_ptr())
    for (M, N, K, bits) in [(64, 4096, 4096, 4), (3, 40, 8192, 2)]:
        banner(f"static split-K M={M} N={N} K={K} bits={bits}")
        A, Bv, Bp, s = _make(bits, M, N, K, seed=M + N + bits)
        Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
        need = bq.gemm_splitk_workspace_bytes(M, N, K, bits)
        assert 0 < need <= 4096 + 256 * 16384
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        ref32 = torch.empty((M, N), dtype=torch.int32, device=dev)
        ref16 = torch.empty((M, N), dtype=torch.float16, device=dev)
        got32 = torch.full((M, N), -1, dtype=torch.int32, device=dev)
        got16 = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        assert L.bq_gemm_splitk(p(Ad), p(Bd), bits, None, p(ref32), M, N, K, p(ws), need, stream) == 0
        assert L.bq_gemm_splitk(p(Ad), p(Bd), bits, p(sd), p(ref16), M, N, K, p(ws), need, stream) == 0
        assert L.bq_gemm_splitk_static(p(Ad), p(Bd), bits, None, p(got32), M, N, K, stream) == 0
        assert L.bq_gemm_splitk_static(p(Ad), p(Bd), bits, p(sd), p(got16), M, N, K, stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(got32, ref32), f"{M}x{N}x{K}: int32 differs from the workspace call"
        assert torch.equal(got16, ref16), f"{M}x{N}x{K}: fp16 differs from the workspace call"
        acc = oracle.gemm_i32(A, Bv)
        assert np.array_equal(got32.cpu().numpy(), acc)
        assert_f16_within_1ulp(f16_bits(got16), oracle.dequant(acc, s), f"static split-K {M}x{N}x{K}")


def test_calls_leave_device_memory_unchanged(dev):
    """After a first call (which may load the library's code object, the
    static scratch with it), further calls of the allocation-free entry point
    and of the automatic GEMM path change the device's free memory by
    nothing: neither allocates."""
    import torch

    from bit_mixed_precision_amd import bq

    M, N, K = 64, 2048, 4096
    A, Bv, Bp, s = _make(4, M, N, K, seed=3)
    Ad, Bd, sd = to_dev(A, dev), to_dev(Bp, dev), to_dev(s, dev)
    o1 = torch.empty((M, N), dtype=torch.float16, device=dev)
    o2 = torch.empty((M, N), dtype=torch.float16, device=dev)
    bq.gemm_splitk_static(Ad, Bd, 4, sd, out=o1)
    bq.gemm(Ad, Bd, 4, sd, out=o2)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(dev)[0]
    for _ in range(3):
        bq.gemm_splitk_static(Ad, Bd, 4, sd, out=o1)
        bq.gemm(Ad, Bd, 4, sd, out=o2)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info(dev)[0] == free0
    assert torch.equal(o1, o2)
