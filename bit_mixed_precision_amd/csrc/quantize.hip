// Per-row symmetric quantization of an fp16 matrix to int8 codes.
//
// BMINF post-training quantization page ("BMINF的後訓練量化實現"), section
// 實現代碼分析2: the quantize() docstring runs two kernels, a per-row
// absmax reduction giving scale = absmax/127 in fp16, then an elementwise
// copy giving the nearest integer of x/scale as int8.  Here both are one
// kernel: a workgroup owns a row, keeps it in registers, reduces the absmax
// (wavefront shuffles, then LDS across the four wavefronts) and writes the
// codes, so x is read from HBM once.
//
// The code range is [-qmax, qmax]: qmax = 127 for int8 as on the page, and
// qmax = 2^(bits-1) - 1 = 7 or 1 for the int4 and ternary weight formats.
//
// Rounding: the code is the nearest integer to the EXACT quotient x/scale,
// ties to even, clamped to [-qmax, qmax].  Without a division per element:
//   q0 = rint(x * r), r = 1/scale rounded to fp32.
// x and scale are fp16 values (11 significant bits), so a quotient that is
// not exactly a half-integer lies at least 2^-13 from every half-integer,
// while x*r is within 190 * 2^-23 of the quotient; q0 is then exact.  For
// an exact half-integer (a tie) the residual e = x - q0*scale, computed
// exactly by one fma (q0*scale has at most 19 significant bits), equals
// +-scale/2, and q0 is moved to the even neighbour if it is odd (the vector
// paths do this in float: q0 + copysign(1/2, e) is then exactly the tie and
// its round-to-nearest-even is the even neighbour).
// The scale itself is fp16(absmax / qmax): fp32 division rounded once more
// to fp16 equals the correctly rounded quotient for every fp16 absmax (a
// quotient that is not exactly an fp16 midpoint lies at least 2^-12 / qmax
// relative from one, far outside fp32 precision; checked exhaustively for
// qmax = 127, 7 and 1).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"

namespace bq {
namespace {

constexpr int kThreads = 256;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t absmax2(uint32_t acc, uint32_t w)
{
    // |x| of fp16 data orders like its magnitude bits as unsigned integers.
    u16x2 a = __builtin_bit_cast(u16x2, acc);
    u16x2 b = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return __half2float(__ushort_as_half((unsigned short)h));
}

__device__ __forceinline__ int code_of(float x, float s, float r, float hs, int qmax)
{
    float q0 = __builtin_rintf(x * r);
    float e = __builtin_fmaf(-q0, s, x);
    int q = (int)q0;
    if (__builtin_fabsf(e) == hs && (q & 1))
        q += (e > 0.f) ? 1 : -1;
    return min(max(q, -qmax), qmax);
}

// Row absmax over the workgroup; every thread gets the result.
__device__ __forceinline__ uint32_t block_absmax(uint32_t m, uint32_t *red)
{
    for (int off = 32; off > 0; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        red[wave] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    return m;
}

struct RowScale {
    float s, r, hs;
    int qmax;
    bool zero;
};

__device__ __forceinline__ RowScale row_scale(uint32_t amax_bits, int qmax, uint16_t *scale_out)
{
    const float a = half_bits_to_float(amax_bits);
    const __half sh = __float2half_rn(__fdiv_rn(a, (float)qmax));
    if (threadIdx.x == 0)
        *scale_out = __half_as_ushort(sh);
    RowScale rs;
    rs.s = __half2float(sh);
    rs.zero = (rs.s == 0.0f);
    rs.r = rs.zero ? 0.0f : __fdiv_rn(1.0f, rs.s);
    rs.hs = 0.5f * rs.s;
    rs.qmax = qmax;
    return rs;
}

// The code plus 128 as a float (an exact integer in [128 - qmax, 128 + qmax]),
// for the vector paths: the tie fix of code_of done in float.  At an exact
// tie the residual e is +-s/2 and q0 + copysign(1/2, e) is exactly the
// half-integer x/s, whose round-to-nearest-even is the even neighbour; off a
// tie the adjustment is 0 and q0 is the code.
__device__ __forceinline__ float code_plus_128(float x, const RowScale &rs)
{
    const float q0 = __builtin_rintf(x * rs.r);
    const float e = __builtin_fmaf(-q0, rs.s, x);
    const float adj = (__builtin_fabsf(e) == rs.hs) ? __builtin_copysignf(0.5f, e) : 0.0f;
    const float q = __builtin_rintf(q0 + adj) + 128.0f;
    return __builtin_amdgcn_fmed3f(q, 128.0f - (float)rs.qmax, 128.0f + (float)rs.qmax);
}

// Four fp16 values (two dwords) -> their four int8 codes (byte i = value i):
// each code + 128 is converted into its byte (v_cvt_pk_u8_f32, exact for
// these integers) and the bias removed from all four at once (code + 128 xor
// 0x80 is the code's two's complement byte).
__device__ __forceinline__ uint32_t codes4(uint32_t w0, uint32_t w1, const RowScale &rs)
{
    uint32_t o = 0;
    o = __builtin_amdgcn_cvt_pk_u8_f32(code_plus_128(half_bits_to_float(w0 & 0xFFFF), rs), 0, o);
    o = __builtin_amdgcn_cvt_pk_u8_f32(code_plus_128(half_bits_to_float(w0 >> 16), rs), 1, o);
    o = __builtin_amdgcn_cvt_pk_u8_f32(code_plus_128(half_bits_to_float(w1 & 0xFFFF), rs), 2, o);
    o = __builtin_amdgcn_cvt_pk_u8_f32(code_plus_128(half_bits_to_float(w1 >> 16), rs), 3, o);
    return o ^ 0x80808080u;
}

// Vector path: cols % 8 == 0, so a row is whole 16-byte vectors of 8 fp16
// and its codes whole 8-byte words.  Thread t owns vectors t, t+256, ...
// (consecutive threads read consecutive 16 bytes).  VPT vectors per thread
// cover rows of up to 2048*VPT elements, held in registers.
template <int VPT>
__global__ __launch_bounds__(kThreads) void quantize_rows_vec(
    const uint4 *__restrict__ x, int64_t cols, int qmax, uint2 *__restrict__ q,
    uint16_t *__restrict__ scale)
{
    __shared__ uint32_t red[4];
    const int64_t row = blockIdx.x;
    const int nvec = (int)(cols >> 3);
    const uint4 *xr = x + row * nvec;
    uint2 *qr = q + row * nvec;

    uint4 v[VPT];
    uint32_t m2 = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int idx = threadIdx.x + j * kThreads;
        v[j] = (idx < nvec) ? load_nt16(xr + idx) : make_uint4(0, 0, 0, 0);
        m2 = absmax2(m2, v[j].x);
        m2 = absmax2(m2, v[j].y);
        m2 = absmax2(m2, v[j].z);
        m2 = absmax2(m2, v[j].w);
    }
    const uint32_t amax = block_absmax(max(m2 & 0xFFFF, m2 >> 16), red);
    const RowScale rs = row_scale(amax, qmax, scale + row);

#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int idx = threadIdx.x + j * kThreads;
        if (idx < nvec) {
            uint2 out = make_uint2(0, 0);
            if (!rs.zero) {
                out.x = codes4(v[j].x, v[j].y, rs);
                out.y = codes4(v[j].z, v[j].w, rs);
            }
            // nontemporal: the codes are not read again by this kernel
            // (measured 31.7 -> 29.5 us for 12288 x 4096 back to back)
            __builtin_nontemporal_store(out.x, &qr[idx].x);
            __builtin_nontemporal_store(out.y, &qr[idx].y);
        }
    }
}

// General path for any cols (and rows too long for registers): two passes
// over the row, the second normally served from L2.
__global__ __launch_bounds__(kThreads) void quantize_rows_any(
    const uint16_t *__restrict__ x, int64_t cols, int qmax, int8_t *__restrict__ q,
    uint16_t *__restrict__ scale)
{
    __shared__ uint32_t red[4];
    const int64_t row = blockIdx.x;
    const uint16_t *xr = x + row * cols;
    int8_t *qr = q + row * cols;
    uint32_t m = 0;
    for (int64_t k = threadIdx.x; k < cols; k += kThreads)
        m = max(m, (uint32_t)(xr[k] & 0x7FFF));
    const uint32_t amax = block_absmax(m, red);
    const RowScale rs = row_scale(amax, qmax, scale + row);
    for (int64_t k = threadIdx.x; k < cols; k += kThreads)
        qr[k] = rs.zero ? 0 : (int8_t)code_of(half_bits_to_float(xr[k]), rs.s, rs.r, rs.hs, rs.qmax);
}

// Fused quantize + pack (int4 / ternary weight preparation): the codes of
// the row rule above with qmax = 7 or 1, written straight in the packed
// storage of bq_pack_int4 / bq_pack_int2 (BitBLAS custom-operator guide,
// cases 1-2: int4 two per byte, low nibble = even k; int2 code v+2 four per
// byte, lowest bits = lowest k), so the int8 codes never go to memory.

// Four int8 codes (byte i = code of k = i) -> their packed bits in the low
// 16 (int4) or 8 (int2) bits.
template <int BITS>
__device__ __forceinline__ uint32_t pack4(uint32_t c)
{
    if constexpr (BITS == 4) {
        const uint32_t n = c & 0x0F0F0F0Fu;  // two's complement nibbles
        const uint32_t t = n | (n >> 4);    // byte 0: k0 | k1 << 4, byte 2: k2 | k3 << 4
        return (t & 0xFFu) | ((t >> 8) & 0xFF00u);
    } else {
        const uint32_t x = (c & 0x03030303u) ^ 0x02020202u;  // code v + 2 (v in [-2, 1])
        return (x | (x >> 6) | (x >> 12) | (x >> 18)) & 0xFFu;
    }
}

// Vector path: cols % 8 == 0; thread t owns 8-element vectors t, t+256, ...
// and writes their 4 (int4) or 2 (int2) packed bytes.
template <int VPT, int BITS>
__global__ __launch_bounds__(kThreads) void quantize_pack_vec(
    const uint4 *__restrict__ x, int64_t cols, uint8_t *__restrict__ packed, uint16_t *__restrict__ scale)
{
    __shared__ uint32_t red[4];
    const int64_t row = blockIdx.x;
    const int nvec = (int)(cols >> 3);
    const uint4 *xr = x + row * nvec;
    constexpr int qmax = (1 << (BITS - 1)) - 1;

    uint4 v[VPT];
    uint32_t m2 = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int idx = threadIdx.x + j * kThreads;
        v[j] = (idx < nvec) ? load_nt16(xr + idx) : make_uint4(0, 0, 0, 0);
        m2 = absmax2(m2, v[j].x);
        m2 = absmax2(m2, v[j].y);
        m2 = absmax2(m2, v[j].z);
        m2 = absmax2(m2, v[j].w);
    }
    const uint32_t amax = block_absmax(max(m2 & 0xFFFF, m2 >> 16), red);
    const RowScale rs = row_scale(amax, qmax, scale + row);

#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int idx = threadIdx.x + j * kThreads;
        if (idx < nvec) {
            const uint32_t c0 = rs.zero ? 0u : codes4(v[j].x, v[j].y, rs);
            const uint32_t c1 = rs.zero ? 0u : codes4(v[j].z, v[j].w, rs);
            if constexpr (BITS == 4) {
                uint32_t *dst = (uint32_t *)(packed + row * (cols >> 1)) + idx;
                __builtin_nontemporal_store(pack4<4>(c0) | (pack4<4>(c1) << 16), dst);
            } else {
                uint16_t *dst = (uint16_t *)(packed + row * (cols >> 2)) + idx;
                __builtin_nontemporal_store((uint16_t)(pack4<2>(c0) | (pack4<2>(c1) << 8)), dst);
            }
        }
    }
}

// General path (cols a multiple of 8 / BITS only): thread t owns packed
// bytes t, t+256, ...; the row is read twice (absmax, then codes).
template <int BITS>
__global__ __launch_bounds__(kThreads) void quantize_pack_any(
    const uint16_t *__restrict__ x, int64_t cols, uint8_t *__restrict__ packed, uint16_t *__restrict__ scale)
{
    __shared__ uint32_t red[4];
    constexpr int qmax = (1 << (BITS - 1)) - 1;
    constexpr int per = 8 / BITS;  // codes per byte
    const int64_t row = blockIdx.x;
    const uint16_t *xr = x + row * cols;
    uint32_t m = 0;
    for (int64_t k = threadIdx.x; k < cols; k += kThreads)
        m = max(m, (uint32_t)(xr[k] & 0x7FFF));
    const uint32_t amax = block_absmax(m, red);
    const RowScale rs = row_scale(amax, qmax, scale + row);
    const int64_t nbytes = cols / per;
    uint8_t *pr = packed + row * nbytes;
    for (int64_t b = threadIdx.x; b < nbytes; b += kThreads) {
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < per; ++j) {
            const int q = rs.zero ? 0 : code_of(half_bits_to_float(xr[b * per + j]), rs.s, rs.r, rs.hs, rs.qmax);
            c |= (uint32_t)(q & 0xFF) << (8 * j);
        }
        pr[b] = (uint8_t)pack4<BITS>(c);
    }
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int qmax,
                                int8_t *q, uint16_t *scale, hipStream_t s)
{
    if (rows == 0)
        return hipSuccess;
    if (!grid_fits(rows, kThreads))
        return kGridTooLarge;
    const dim3 grid((unsigned)rows), block(kThreads);
    const int64_t nvec = cols / 8;
    const bool vec = (cols % 8 == 0) && cols > 0;
    if (vec && nvec <= 1 * kThreads)
        quantize_rows_vec<1><<<grid, block, 0, s>>>((const uint4 *)x, cols, qmax, (uint2 *)q, scale);
    else if (vec && nvec <= 2 * kThreads)
        quantize_rows_vec<2><<<grid, block, 0, s>>>((const uint4 *)x, cols, qmax, (uint2 *)q, scale);
    else if (vec && nvec <= 4 * kThreads)
        quantize_rows_vec<4><<<grid, block, 0, s>>>((const uint4 *)x, cols, qmax, (uint2 *)q, scale);
    else if (vec && nvec <= 8 * kThreads)
        quantize_rows_vec<8><<<grid, block, 0, s>>>((const uint4 *)x, cols, qmax, (uint2 *)q, scale);
    else
        quantize_rows_any<<<grid, block, 0, s>>>(x, cols, qmax, q, scale);
    return hipGetLastError();
}

}  // namespace bq

namespace bq {

hipError_t launch_quantize_pack(const uint16_t *x, int64_t rows, int64_t cols, int bits, uint8_t *packed,
                                uint16_t *scale, hipStream_t s)
{
    if (rows == 0)
        return hipSuccess;
    if (!grid_fits(rows, kThreads))
        return kGridTooLarge;
    const dim3 grid((unsigned)rows), block(kThreads);
    const int64_t nvec = cols / 8;
    const bool vec = (cols % 8 == 0) && cols > 0 && nvec <= 8 * kThreads;
#define BQ_QP(BITS_)                                                                                    \
    if (!vec)                                                                                           \
        quantize_pack_any<BITS_><<<grid, block, 0, s>>>(x, cols, packed, scale);                       \
    else if (nvec <= kThreads)                                                                          \
        quantize_pack_vec<1, BITS_><<<grid, block, 0, s>>>((const uint4 *)x, cols, packed, scale);     \
    else if (nvec <= 2 * kThreads)                                                                      \
        quantize_pack_vec<2, BITS_><<<grid, block, 0, s>>>((const uint4 *)x, cols, packed, scale);     \
    else if (nvec <= 4 * kThreads)                                                                      \
        quantize_pack_vec<4, BITS_><<<grid, block, 0, s>>>((const uint4 *)x, cols, packed, scale);     \
    else                                                                                                \
        quantize_pack_vec<8, BITS_><<<grid, block, 0, s>>>((const uint4 *)x, cols, packed, scale);
    if (bits == 4) {
        BQ_QP(4)
    } else {
        BQ_QP(2)
    }
#undef BQ_QP
    return hipGetLastError();
}

}  // namespace bq
