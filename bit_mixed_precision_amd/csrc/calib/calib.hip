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
