// Internal declarations shared by the HIP translation units of libbq.so.
// Not installed; the public interface is include/bq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gelu_fit.h"

namespace bq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint (data read once: streamed weights
// and activations that should not displace reused lines in the caches).
__device__ __forceinline__ uint4 load_nt16(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A dispatch counts work-items, not workgroups, per grid dimension, and the
// count must stay below 2^32.  Launchers check their grid with grid_fits and
// return kGridTooLarge (reported as a shape error by the C ABI) instead of
// launching when it does not.
constexpr hipError_t kGridTooLarge = hipErrorInvalidConfiguration;
inline bool grid_fits(int64_t workgroups, int threads) { return workgroups * threads < (1LL << 32); }

// Kernel launchers.  Arguments have been validated by the C ABI layer:
// sizes are non-negative and within limits, pointers non-null and aligned.
// Each returns the status of the launch (hipGetLastError after it).
// Codes in [-qmax, qmax], scale = fp16(absmax / qmax); 1 <= qmax <= 127.
hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int qmax,
                                int8_t *q, uint16_t *scale, hipStream_t s);
// The codes of launch_quantize_rows with qmax = 7 (bits 4) or 1 (bits 2),
// written packed like launch_pack_int4 / launch_pack_int2; cols % (8 / bits) == 0.
hipError_t launch_quantize_pack(const uint16_t *x, int64_t rows, int64_t cols, int bits, uint8_t *packed,
                                uint16_t *scale, hipStream_t s);
hipError_t launch_pack_int4(const int8_t *v, int64_t total, uint8_t *out, hipStream_t s);
hipError_t launch_pack_int2(const int8_t *v, int64_t total, uint8_t *out, hipStream_t s);

// GELU(v) = v * Phi(v) in fp32 with the constants of gelu_fit.h (from
// gen_gelu_fit.py): Phi(v) = 1 - H for v >= 0 and H for v < 0, where
// H = erfc(|v| / sqrt 2) / 2 = exp2(v^2 kGeluE) Q(t), t = 1 / (1 + kGeluA |v|),
// Q a degree-4 fit (relative error about 6e-5, eight times below the
// smallest relative fp16 ulp); |v| is clamped to kGeluVmax inside t only.
// About 11 VALU operations and two transcendental ones (rcp, exp2).
__device__ __forceinline__ float gelu_fit(float v)
{
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(kGeluA, fminf(fabsf(v), kGeluVmax), 1.0f));
    float q = kGeluQ[kGeluDeg];
#pragma unroll
    for (int k = kGeluDeg - 1; k >= 0; --k)
        q = __builtin_fmaf(q, t, kGeluQ[k]);
    const float h = __builtin_amdgcn_exp2f(v * v * kGeluE) * q;
    return v * (v >= 0.0f ? 1.0f - h : h);
}

// Activation applied to the dequantized fp32 value before the fp16
// conversion: 0 identity, 1 ReLU, 2 GELU (gelu_fit).  ACT fixed at compile
// time (the tiled GEMM's epilogue), or chosen per call (apply_act).
template <int ACT>
__device__ __forceinline__ float act_fixed(float v)
{
    if constexpr (ACT == 1)
        return fmaxf(v, 0.0f);
    else if constexpr (ACT == 2)
        return gelu_fit(v);
    else
        return v;
}

__device__ __forceinline__ float apply_act(float v, int act)
{
    return act == 1 ? act_fixed<1>(v) : act == 2 ? act_fixed<2>(v) : v;
}

// Per-batch element strides of a batched GEMM launch (grid dimension y is the
// batch index z): batch z uses A + z*a, B + z*b (bytes of packed B),
// scale + z*s and C + z*c (elements of the output type).  The activation
// scale, when given, is shared by all batches.
struct BatchStrides {
    int64_t a = 0, b = 0, s = 0, c = 0;
};

// The GEMM launchers: scale == nullptr selects the int32 output; with an fp16
// output, xscale (nullable) holds a per-row activation scale [M] that
// multiplies the weight scale, and act (apply_act) is applied before the
// conversion.
// Decode GEMV on the dot-product ALUs, M <= 4.
hipError_t launch_gemv(const int8_t *A, const uint8_t *B, int bits, const uint16_t *scale,
                       const uint16_t *xscale, int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s);
// Streaming matrix-core GEMM (operands through per-wavefront LDS-DMA chunk
// buffers, K split over the wavefronts of a workgroup), M <= 256.
hipError_t launch_gemm_stream(const int8_t *A, const uint8_t *B, int bits,
                              const uint16_t *scale, const uint16_t *xscale, int act, void *C,
                              int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s);
// LDS-tiled matrix-core GEMM, any M.  With a workspace (ws, wsBytes) of at
// least gemm_splitk_workspace_bytes(M, N, K, bits) bytes whose first 4 KiB
// are zero, a shape with few output tiles splits K over workgroups; without
// one (ws == nullptr) K is never split.
hipError_t launch_gemm_tiled(const int8_t *A, const uint8_t *B, int bits,
                             const uint16_t *scale, const uint16_t *xscale, int act, void *C,
                             int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s,
                             void *ws = nullptr, int64_t wsBytes = 0);
// Workspace bytes the tiled GEMM uses to split K for this shape (0: no split).
int64_t gemm_splitk_workspace_bytes(int M, int N, int K, int bits);
// W4A16 GEMM with NF4 weight codes on the tiled kernel: A fp16 [M, K], B
// codes [N, K/2], per-row scale and zero point (zero may be NULL), C fp16.
hipError_t launch_gemm_nf4(const uint16_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *zero,
                           uint16_t *C, int M, int N, int K, hipStream_t s);
// The same product for M <= 4 as a stream over B (decode).
hipError_t launch_gemv_nf4(const uint16_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *zero,
                           uint16_t *C, int M, int N, int K, hipStream_t s);

}  // namespace bq
