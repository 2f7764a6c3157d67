// Measurement kernels for the benchmark's achievable ceilings on the box it
// runs on (not part of the library's interface, include/bq.h): a loop of
// int8 matrix-core instructions on register operands only, and a plain
// streaming read of a device buffer.  Their rates are the "achievable" bounds
// reported beside the published peaks (8 TB/s HBM, 5.0 POP/s dense int8).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {
namespace calib {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Every wavefront runs `iters` rounds of four independent
// v_mfma_i32_32x32x32_i8 (4 x 65536 int8 operations per round); one value
// per thread is stored so the work is not optimized away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, int *__restrict__ out)
{
    const v4i a = {(int)threadIdx.x, 0x01020304, 0x05060708, (int)blockIdx.x};
    const v4i b = {0x7F7F7F7F, (int)threadIdx.x * 3, 0x10203040, 0x0A0B0C0D};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        s ^= c0[e] + c1[e] + c2[e] + c3[e];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The matrix-core instruction stream of the W4A8 GEMM's 128-k stage with no
// memory traffic, as one wavefront of the M = 4096 kernel issues it: two 64-k
// sub-steps of v_mfma_i32_16x16x64_i8, each 8 A operands x 4 B operands into
// 32 accumulators, A first and each A operand held for four consecutive
// instructions, on operands drawn like the workload's (A bytes uniform in
// [-127, 127], B bytes 16 v with v uniform in [-8, 7], as the kernels feed
// unpacked int4).  The matrix cores' power, and with it the clock they hold,
// depends on the operand bits and on the instruction shape and order;
// constant operands (mfma_loop_kernel) keep the clock far higher than such
// data does.  2^21 operations per wavefront per iteration.
__global__ __launch_bounds__(256) void mfma_w4a8_stream_kernel(int iters, int *__restrict__ out)
{
    uint32_t h = (uint32_t)(blockIdx.x * blockDim.x + threadIdx.x) * 2654435761u + 0x9E3779B9u;
    auto next = [&h]() {  // xorshift32
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        return h;
    };
    v4i a[2][8], b[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t w = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w |= (uint32_t)(uint8_t)(int8_t)((int)(next() % 255u) - 127) << (8 * q);
                a[ks][i][e] = (int)w;
            }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                b[ks][j][e] = (int)(next() & 0xF0F0F0F0u);
    }
    v4i c[8][4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    c[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[ks][i], b[ks][j], c[i][j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s ^= c[i][j][e];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride read of n16 16-byte words with nontemporal loads; each thread
// stores the XOR of what it read.
__global__ __launch_bounds__(256) void read_stream_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ out)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t x = 0;
#pragma unroll 8
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(p + i));
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace calib
}  // namespace bq

extern "C" {

// blocks x 256 threads, `out` holds blocks * 256 ints.  Returns a hipError_t.
int bq_calib_mfma_loop(int blocks, int iters, int *out, void *stream)
{
    if (blocks <= 0 || iters < 0 || !out)
        return (int)hipErrorInvalidValue;
    bq::calib::mfma_loop_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(iters, out);
    return (int)hipGetLastError();
}

// blocks x 256 threads, 32 matrix instructions per iteration per wavefront;
// `out` holds blocks * 256 ints.  Returns a hipError_t.
int bq_calib_mfma_w4a8_stream(int blocks, int iters, int *out, void *stream)
{
    if (blocks <= 0 || iters < 0 || !out)
        return (int)hipErrorInvalidValue;
    bq::calib::mfma_w4a8_stream_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(iters, out);
    return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) from `buf`; blocks x 256
// threads, `out` holds blocks * 256 uint32.  Returns a hipError_t.
int bq_calib_read_stream(const void *buf, int64_t bytes, int blocks, uint32_t *out, void *stream)
{
    if (blocks <= 0 || bytes < 0 || bytes % 16 != 0 || !buf || !out || ((uintptr_t)buf & 15) != 0)
        return (int)hipErrorInvalidValue;
    bq::calib::read_stream_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(
        (const uint4 *)buf, bytes / 16, out);
    return (int)hipGetLastError();
}

}  // extern "C"
