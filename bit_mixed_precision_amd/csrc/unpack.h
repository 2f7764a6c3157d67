// In-register unpacking of packed int4 / int2 weights into signed int8
// matrix-core operands.
//
// Storage (BitBLAS custom-operator guide, cases 1-2; bit order as in
// bq_pack_int4 / bq_pack_int2): int4 two's complement, low nibble = even k;
// int2 code v+2 in bits 2j..2j+1 for k = 4b + j.
//
// Instead of sign-extending each value, the value is placed in the HIGH bits
// of its byte with zeros below, which makes the byte equal to 16*v (int4) or
// 64*v (int2) as a signed int8.  The integer products then sum to 16*acc or
// 64*acc exactly (|16v|, |64v| <= 128 keep the int32 bound of int8 x int8),
// and one arithmetic shift right by 4 or 6 recovers acc.  For int2,
// flipping the high bit of each code (xor 2) turns code v+2 into v as a
// 2-bit two's complement number.
//
// Output order is the natural k order, so A operands need no permutation.
#pragma once

#include <stdint.h>

#include "bq_internal.h"

namespace bq {

// One packed dword (8 int4 values, k = 0..7) -> two dwords holding 16*v for
// k = 0..3 and k = 4..7 (byte i = k i).
__device__ __forceinline__ void unpack8_int4(uint32_t p, uint32_t &o0, uint32_t &o1)
{
    const uint32_t lo = (p << 4) & 0xF0F0F0F0u;  // byte b: even k = 2b, times 16
    const uint32_t hi = p & 0xF0F0F0F0u;         // byte b: odd k = 2b+1, times 16
    // v_perm_b32 selects bytes from {hi:lo} (lo = bytes 0-3, hi = bytes 4-7).
    o0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // lo.b0 hi.b0 lo.b1 hi.b1
    o1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // lo.b2 hi.b2 lo.b3 hi.b3
}

// One packed dword (16 int2 codes, k = 0..15) -> four dwords holding 64*v
// for k = 0..3, 4..7, 8..11, 12..15.
__device__ __forceinline__ void unpack16_int2(uint32_t p, uint32_t &o0, uint32_t &o1,
                                              uint32_t &o2, uint32_t &o3)
{
    const uint32_t x = p ^ 0xAAAAAAAAu;             // code v+2 -> v (2-bit two's complement)
    const uint32_t c0 = (x << 6) & 0xC0C0C0C0u;     // byte b: k = 4b     (times 64)
    const uint32_t c1 = (x << 4) & 0xC0C0C0C0u;     // byte b: k = 4b + 1
    const uint32_t c2 = (x << 2) & 0xC0C0C0C0u;     // byte b: k = 4b + 2
    const uint32_t c3 = x & 0xC0C0C0C0u;            // byte b: k = 4b + 3
    const uint32_t t01a = __builtin_amdgcn_perm(c1, c0, 0x05010400u);  // k 0,1,4,5
    const uint32_t t01b = __builtin_amdgcn_perm(c1, c0, 0x07030602u);  // k 8,9,12,13
    const uint32_t t23a = __builtin_amdgcn_perm(c3, c2, 0x05010400u);  // k 2,3,6,7
    const uint32_t t23b = __builtin_amdgcn_perm(c3, c2, 0x07030602u);  // k 10,11,14,15
    o0 = __builtin_amdgcn_perm(t23a, t01a, 0x05040100u);  // k 0,1,2,3
    o1 = __builtin_amdgcn_perm(t23a, t01a, 0x07060302u);  // k 4,5,6,7
    o2 = __builtin_amdgcn_perm(t23b, t01b, 0x05040100u);  // k 8..11
    o3 = __builtin_amdgcn_perm(t23b, t01b, 0x07060302u);  // k 12..15
}

template <int BITS>
struct Unpack;

// A 16-byte packed chunk -> 16*8/BITS bytes of operand (as dwords).
template <>
struct Unpack<8> {
    static constexpr int kShift = 0;
    static constexpr int kOutDwords = 4;
    // operand t (16 bytes = 16 k) of a 16-byte packed chunk
    template <int TT>
    __device__ __forceinline__ static v4i operand(const uint4 &p)
    {
        static_assert(TT == 0, "one operand per chunk");
        return (v4i){(int)p.x, (int)p.y, (int)p.z, (int)p.w};
    }
    __device__ __forceinline__ static v4i operand_rt(const uint4 &p, int) { return operand<0>(p); }
    __device__ __forceinline__ static void run(const uint4 &p, uint32_t *o)
    {
        o[0] = p.x;
        o[1] = p.y;
        o[2] = p.z;
        o[3] = p.w;
    }
};

template <>
struct Unpack<4> {
    static constexpr int kShift = 4;
    static constexpr int kOutDwords = 8;
    template <int TT>
    __device__ __forceinline__ static v4i operand(const uint4 &p)
    {
        static_assert(TT == 0 || TT == 1, "two operands per chunk");
        uint32_t o0, o1, o2, o3;
        unpack8_int4(TT == 0 ? p.x : p.z, o0, o1);
        unpack8_int4(TT == 0 ? p.y : p.w, o2, o3);
        return (v4i){(int)o0, (int)o1, (int)o2, (int)o3};
    }
    // operand tt (0 or 1) chosen at run time: the two dwords are selected first
    __device__ __forceinline__ static v4i operand_rt(const uint4 &p, int tt)
    {
        uint32_t o0, o1, o2, o3;
        unpack8_int4(tt == 0 ? p.x : p.z, o0, o1);
        unpack8_int4(tt == 0 ? p.y : p.w, o2, o3);
        return (v4i){(int)o0, (int)o1, (int)o2, (int)o3};
    }
    __device__ __forceinline__ static void run(const uint4 &p, uint32_t *o)
    {
        unpack8_int4(p.x, o[0], o[1]);
        unpack8_int4(p.y, o[2], o[3]);
        unpack8_int4(p.z, o[4], o[5]);
        unpack8_int4(p.w, o[6], o[7]);
    }
};

template <>
struct Unpack<2> {
    static constexpr int kShift = 6;
    static constexpr int kOutDwords = 16;
    template <int TT>
    __device__ __forceinline__ static v4i operand(const uint4 &p)
    {
        static_assert(TT >= 0 && TT < 4, "four operands per chunk");
        uint32_t o0, o1, o2, o3;
        unpack16_int2(TT == 0 ? p.x : TT == 1 ? p.y : TT == 2 ? p.z : p.w, o0, o1, o2, o3);
        return (v4i){(int)o0, (int)o1, (int)o2, (int)o3};
    }
    // operand tt (0 .. 3) chosen at run time
    __device__ __forceinline__ static v4i operand_rt(const uint4 &p, int tt)
    {
        uint32_t o0, o1, o2, o3;
        unpack16_int2(tt == 0 ? p.x : tt == 1 ? p.y : tt == 2 ? p.z : p.w, o0, o1, o2, o3);
        return (v4i){(int)o0, (int)o1, (int)o2, (int)o3};
    }
    __device__ __forceinline__ static void run(const uint4 &p, uint32_t *o)
    {
        unpack16_int2(p.x, o[0], o[1], o[2], o[3]);
        unpack16_int2(p.y, o[4], o[5], o[6], o[7]);
        unpack16_int2(p.z, o[8], o[9], o[10], o[11]);
        unpack16_int2(p.w, o[12], o[13], o[14], o[15]);
    }
};

}  // namespace bq
