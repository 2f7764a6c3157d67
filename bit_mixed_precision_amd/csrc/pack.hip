// Packing of int8-held int4 / int2 weight values into bytes along K.
//
// BitBLAS custom-operator guide ("BitBLAS自定义操作开发指南"), case 2:
// 4-bit weights stored compressed as uint8 [N, K/2]; case 1: BitNet-b1.58
// 2-bit weights, here four per byte as uint8 [N, K/4].  Bit order:
//   int4: byte = (v[k] & 0xF) | (v[k+1] & 0xF) << 4        (k even)
//   int2: byte = sum_j ((v[k+j] + 2) & 3) << 2j            (k % 4 == 0)
// K is a multiple of the pack factor, so rows never share a byte and the
// packing is one flat elementwise pass over n*k values.  Memory bound:
// each thread reads 16 values as one 16-byte load and writes 8 / 4 bytes.
#include <hip/hip_runtime.h>

#include "bq_internal.h"

namespace bq {
namespace {

constexpr int kThreads = 256;

// Four int4 values (one per byte of w, lowest byte = lowest k) -> 16 bits.
__device__ __forceinline__ uint32_t pack4_nibbles(uint32_t w)
{
    return (w & 0xFu) | ((w >> 4) & 0xF0u) | ((w >> 8) & 0xF00u) | ((w >> 12) & 0xF000u);
}

// Four int2 values (one per byte of w) -> 8 bits of codes v+2.
__device__ __forceinline__ uint32_t pack4_crumbs(uint32_t w)
{
    const uint32_t c = (w & 0x03030303u) ^ 0x02020202u;  // (v + 2) mod 4 per byte
    return (c & 0x3u) | ((c >> 6) & 0xCu) | ((c >> 12) & 0x30u) | ((c >> 18) & 0xC0u);
}

__global__ __launch_bounds__(kThreads) void pack_int4_kernel(
    const uint4 *__restrict__ v, int64_t nvec, uint2 *__restrict__ out,
    const int8_t *__restrict__ tail_v, int64_t tail, uint8_t *__restrict__ tail_out)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        const uint4 w = load_nt16(v + i);
        uint2 o;
        o.x = pack4_nibbles(w.x) | (pack4_nibbles(w.y) << 16);
        o.y = pack4_nibbles(w.z) | (pack4_nibbles(w.w) << 16);
        out[i] = o;
    }
    // Fewer than 16 trailing values (an even count): one thread per pair.
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t < tail / 2)
        tail_out[t] = (uint8_t)((tail_v[2 * t] & 0xF) | ((tail_v[2 * t + 1] & 0xF) << 4));
}

__global__ __launch_bounds__(kThreads) void pack_int2_kernel(
    const uint4 *__restrict__ v, int64_t nvec, uint32_t *__restrict__ out,
    const int8_t *__restrict__ tail_v, int64_t tail, uint8_t *__restrict__ tail_out)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        const uint4 w = load_nt16(v + i);
        out[i] = pack4_crumbs(w.x) | (pack4_crumbs(w.y) << 8) |
                 (pack4_crumbs(w.z) << 16) | (pack4_crumbs(w.w) << 24);
    }
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t < tail / 4) {
        uint32_t w = 0;
        for (int j = 0; j < 4; ++j)
            w |= (uint32_t)(uint8_t)tail_v[4 * t + j] << (8 * j);
        tail_out[t] = (uint8_t)pack4_crumbs(w);
    }
}

unsigned grid_for(int64_t nvec)
{
    // Enough workgroups for ~8 per CU on 256 CUs, fewer for small inputs.
    int64_t g = (nvec + kThreads - 1) / kThreads;
    if (g > 2048)
        g = 2048;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_pack_int4(const int8_t *v, int64_t total, uint8_t *out, hipStream_t s)
{
    if (total == 0)
        return hipSuccess;
    const int64_t nvec = total / 16, tail = total % 16;
    pack_int4_kernel<<<grid_for(nvec), kThreads, 0, s>>>(
        (const uint4 *)v, nvec, (uint2 *)out, v + nvec * 16, tail, out + nvec * 8);
    return hipGetLastError();
}

hipError_t launch_pack_int2(const int8_t *v, int64_t total, uint8_t *out, hipStream_t s)
{
    if (total == 0)
        return hipSuccess;
    const int64_t nvec = total / 16, tail = total % 16;
    pack_int2_kernel<<<grid_for(nvec), kThreads, 0, s>>>(
        (const uint4 *)v, nvec, (uint32_t *)out, v + nvec * 16, tail, out + nvec * 4);
    return hipGetLastError();
}

}  // namespace bq
