// Global -> LDS loads without registers (the LDS-DMA form of the 16-byte
// buffer load) and the wait-count helpers that go with them; shared by the
// matrix-core GEMM kernels of libbq.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int v4si __attribute__((ext_vector_type(4)));

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset that is always out of range

// Raw buffer resource (gfx9 layout): base address, stride 0, byte range,
// default format word.  Offsets at or past `bytes` read as zero.
__device__ __forceinline__ v4si make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    return (v4si){(int)(uint32_t)a, (int)((a >> 32) & 0xFFFF), (int)bytes, 0x00020000};
}

// LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(lds_void_t *)p;
}

// 16-byte buffer load written straight to LDS: lane i stores its 16 bytes at
// LDS address lds_addr + 16 i.  Issued as inline assembly so the compiler's
// wait-count pass does not order every later LDS read behind it; the kernels
// wait for these loads explicitly (wait_vmcnt) before the LDS is read.
__device__ __forceinline__ void dma16(v4si rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr));
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// s_waitcnt with only the LDS / scalar-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_lgkmcnt()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

// wait_vmcnt<F * c>() for a wave-uniform c in [0, C] (the counter limit must
// be an immediate, so one branch per value).
template <int F, int C>
__device__ __forceinline__ void wait_vmcnt_rt(int c)
{
    if constexpr (C > 0) {
        if (c == C) {
            wait_vmcnt<F * C>();
            return;
        }
        wait_vmcnt_rt<F, C - 1>(c);
    } else {
        wait_vmcnt<0>();
    }
}

}  // namespace bq
