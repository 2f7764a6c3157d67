// Decoding of 4-bit NormalFloat (NF4) weight codes from a per-lane register
// table (BitBLAS custom-operator guide, case 2: W4A16 with NF4 weights);
// shared by the NF4 decode GEMV and the NF4 mode of the tiled GEMM.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bq_internal.h"
#include "nf4_table.h"

namespace bq {

// One B row's 16 dequantized fp16 weights: the low bytes of entries
// 4q..4q+3 in lo[q], the high bytes in hi[q].  A byte permute
// (v_perm_b32) selects among 8 table bytes per output byte, so entries 0-7
// and 8-15 are selected separately and merged by the code's bit 3: no LDS
// lookups (and no bank conflicts) on the way to the arithmetic.
struct Nf4Lut {
    uint32_t lo[4], hi[4];
};

// The table of the row with fp16 scale and zero point bits: entry c is
// fp16(fp32(table[c] - zero) * scale), two fp32 roundings then one to fp16.
// The empty asm keeps the product a value of its own, so the compiler cannot
// fuse the multiply with the conversion (one rounding of the exact product).
__device__ __forceinline__ Nf4Lut nf4_lut(uint16_t scaleBits, uint16_t zeroBits)
{
    const float s = __half2float(__ushort_as_half(scaleBits));
    const float z = __half2float(__ushort_as_half(zeroBits));
    Nf4Lut t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float d = __half2float(__ushort_as_half(kNf4TableF16[4 * q + e])) - z;
            float w = d * s;
            asm volatile("" : "+v"(w));
            const uint32_t h = __half_as_ushort(__float2half_rn(w));
            lo |= (h & 0xFFu) << (8 * e);
            hi |= (h >> 8) << (8 * e);
        }
        t.lo[q] = lo;
        t.hi[q] = hi;
    }
    return t;
}

// Four codes (one per byte, 0..15) -> their four fp16 weights, two per dword
// in byte order (the code in byte 0 in the low half of o01).
__device__ __forceinline__ void nf4_lookup4(uint32_t c, const Nf4Lut &t, uint32_t &o01, uint32_t &o23)
{
    const uint32_t sel = c & 0x07070707u;
    const uint32_t m8 = c & 0x08080808u;
    const uint32_t mask = (m8 << 5) - (m8 >> 3);  // 0xFF in the bytes whose code is >= 8
    const uint32_t lo0 = __builtin_amdgcn_perm(t.lo[1], t.lo[0], sel);
    const uint32_t lo1 = __builtin_amdgcn_perm(t.lo[3], t.lo[2], sel);
    const uint32_t hi0 = __builtin_amdgcn_perm(t.hi[1], t.hi[0], sel);
    const uint32_t hi1 = __builtin_amdgcn_perm(t.hi[3], t.hi[2], sel);
    const uint32_t lo = (lo1 & mask) | (lo0 & ~mask);
    const uint32_t hi = (hi1 & mask) | (hi0 & ~mask);
    o01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // lo.b0 hi.b0 lo.b1 hi.b1
    o23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // lo.b2 hi.b2 lo.b3 hi.b3
}

// Eight 4-bit codes (one dword, the lowest k in the low nibble) -> eight
// fp16 weights of one B row, in k order.
__device__ __forceinline__ v4i decode_nf4(uint32_t p, const Nf4Lut &t)
{
    const uint32_t ev = p & 0x0F0F0F0Fu;                               // codes of k = 0, 2, 4, 6
    const uint32_t od = (p >> 4) & 0x0F0F0F0Fu;                        // k = 1, 3, 5, 7
    const uint32_t c03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);  // k = 0, 1, 2, 3
    const uint32_t c47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);  // k = 4, 5, 6, 7
    uint32_t o[4];
    nf4_lookup4(c03, t, o[0], o[1]);
    nf4_lookup4(c47, t, o[2], o[3]);
    return (v4i){(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

}  // namespace bq
