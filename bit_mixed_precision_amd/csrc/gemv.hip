// Decode GEMV (M <= 4): acc[m,n] = sum_k A[m,k] * B[n,k], optionally
// C = fp16(acc * scale[n]) (BitBLAS custom-operator guide, sections 1-2 and
// case 1; the decode-step linear layers of the BMINF page, section
// 實現代碼分析2, whose activations are one token row per sequence).
//
// At M <= 4 every byte of B feeds at most 4 multiply-adds, so the kernel is a
// stream over B and its time is the time to pull B out of HBM plus the fixed
// cost of a launch.  It is laid out like a plain streaming read, with as
// little as possible on either side of the stream:
//  * one wavefront per R consecutive rows of B; its 64 lanes walk each packed
//    row in 16-byte chunks (lane l takes chunks l, l + 64, ...), so one load
//    instruction covers 1 KB of a row;
//  * the bytes of A a pass multiplies are the same for every wavefront of
//    the workgroup: wavefront 0 brings them into LDS with the LDS-DMA form
//    of the 16-byte buffer load (1 KB of consecutive bytes per instruction),
//    and after a barrier every lane reads its slice from there; every B load
//    of a lane (its chunks of all R rows) is issued before any is used, and
//    the weight scale of the output the lane writes just before them, so no
//    memory latency follows the stream;
//  * packed values are unpacked in registers to 16 v / 64 v bytes with
//    shifts and masks only, the A bytes permuted to match once per chunk for
//    all R rows, and multiplied with v_dot4_i32_i8;
//  * the R x MR lane sums are reduced across the wavefront by a butterfly that
//    halves the number of values at each of the first log2(R MR) steps (each
//    lane keeps the half its partner does not, and adds the partner's copy of
//    it), so R MR sums cost R MR - 1 + 6 - log2(R MR) exchanges instead of
//    6 R MR, those within a 16-lane row as DPP operands of the adds; the
//    lane that ends with sum (m, r) writes that output.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "lds_dma.h"
#include "unpack.h"

namespace bq {
namespace {

// Sum over the 16 lanes of a row of the wavefront, every lane of the row
// receiving it: row mirror (lane i with 15 - i), half-row mirror (i with
// 7 - i within each 8), then the two pair swaps of a quad, as DPP operands.
__device__ __forceinline__ int row_sum16(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
    return v;
}

// Packed B bytes of one 16-byte chunk as dot-product operands, without the
// byte permutes that would restore k order (the A bytes are permuted to
// match instead, once per chunk for all the rows of a wavefront).  Values sit
// in the high bits of their bytes (16 v for int4, 64 v for int2, as in
// unpack.h), so each product is exact and the sums are 2^kShift times the
// true ones:
//  * int4, dword d of the chunk (k = 8d ... 8d + 7): o[2d] byte b holds
//    k = 8d + 2b, o[2d + 1] byte b holds k = 8d + 2b + 1;
//  * int2, dword d (k = 16d ... 16d + 15): o[4d + j] byte b holds
//    k = 16d + 4b + j (code v + 2 turned into v by flipping its high bit);
//  * int8: the bytes as they are.
template <int BITS>
__device__ __forceinline__ void unpack_b(const uint4 &p, uint32_t *o)
{
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (BITS == 8) {
            o[d] = w[d];
        } else if constexpr (BITS == 4) {
            o[2 * d] = (w[d] << 4) & 0xF0F0F0F0u;
            o[2 * d + 1] = w[d] & 0xF0F0F0F0u;
        } else {
            const uint32_t x = w[d] ^ 0xAAAAAAAAu;
            o[4 * d] = (x << 6) & 0xC0C0C0C0u;
            o[4 * d + 1] = (x << 4) & 0xC0C0C0C0u;
            o[4 * d + 2] = (x << 2) & 0xC0C0C0C0u;
            o[4 * d + 3] = x & 0xC0C0C0C0u;
        }
    }
}

// The A bytes of a 16-byte packed B chunk (16 * 8 / BITS of them, in k
// order) rearranged to pair with unpack_b's operands.
template <int BITS>
__device__ __forceinline__ void order_a(const uint4 *a, uint32_t *ap)
{
    constexpr int kD = 16 * 8 / BITS / 4;  // A dwords per chunk
    uint32_t w[kD];
#pragma unroll
    for (int h = 0; h < kD / 4; ++h) {
        w[4 * h] = a[h].x, w[4 * h + 1] = a[h].y, w[4 * h + 2] = a[h].z, w[4 * h + 3] = a[h].w;
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (BITS == 8) {
            ap[d] = w[d];
        } else if constexpr (BITS == 4) {
            // even k (8d, 8d + 2, 8d + 4, 8d + 6) and odd k of A dwords 2d, 2d + 1
            ap[2 * d] = __builtin_amdgcn_perm(w[2 * d + 1], w[2 * d], 0x06040200u);
            ap[2 * d + 1] = __builtin_amdgcn_perm(w[2 * d + 1], w[2 * d], 0x07050301u);
        } else {
            // 4 x 4 byte transpose of A dwords 4d .. 4d + 3: ap[4d + j] byte b
            // = A[16d + 4b + j]
            const uint32_t t0 = __builtin_amdgcn_perm(w[4 * d + 1], w[4 * d], 0x05010400u);
            const uint32_t t1 = __builtin_amdgcn_perm(w[4 * d + 1], w[4 * d], 0x07030602u);
            const uint32_t t2 = __builtin_amdgcn_perm(w[4 * d + 3], w[4 * d + 2], 0x05010400u);
            const uint32_t t3 = __builtin_amdgcn_perm(w[4 * d + 3], w[4 * d + 2], 0x07030602u);
            ap[4 * d] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
            ap[4 * d + 1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
            ap[4 * d + 2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
            ap[4 * d + 3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
        }
    }
}

// MR rows of A, R rows of B per wavefront, WAVES wavefronts per workgroup,
// U chunks per lane per row per pass (U * 1 KB of each row per pass).
template <int BITS, int MR, int R, int WAVES, int U, bool F16OUT>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(
    const int8_t *__restrict__ A, const uint8_t *__restrict__ B,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ xscale, int act,
    void *__restrict__ C, int M, int N, int K, BatchStrides bs)
{
    constexpr int kV = MR * R;  // sums per lane
    static_assert((kV & (kV - 1)) == 0 && kV <= 64, "a power of two of sums per wavefront");
    constexpr int kLogV = kV >= 64 ? 6 : kV >= 32 ? 5 : kV >= 16 ? 4 : kV >= 8 ? 3 : kV >= 4 ? 2 : kV >= 2 ? 1 : 0;
    if (gridDim.y > 1) {  // batch blockIdx.y (BatchStrides)
        const int64_t z = blockIdx.y;
        A += z * bs.a;
        B += z * bs.b;
        if (F16OUT) {
            scale += z * bs.s;
            C = (uint16_t *)C + z * bs.c;
        } else {
            C = (int *)C + z * bs.c;
        }
    }
    using Up = Unpack<BITS>;
    constexpr int kAPerChunk = 16 * 8 / BITS;  // bytes of A (= k values) per packed chunk
    constexpr int kAPass = 64 * U * kAPerChunk;  // bytes of one A row per pass (4 KB)
    static_assert(kAPass % 1024 == 0, "whole 1 KB DMA blocks");
    // the A bytes of a pass, two passes deep: the same for every wavefront
    __shared__ __attribute__((aligned(1024))) uint8_t As[2][MR][kAPass];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = (blockIdx.x * WAVES + wave) * R;
    const int64_t rowBytes = (int64_t)K * BITS / 8;
    const int chunks = (int)(rowBytes / 16);  // K % 64 == 0: whole chunks
    // a wavefront past N loads and stores nothing but takes part in every
    // barrier (wavefront 0, which moves A, is never past N)
    if (n0 >= N) {
        for (int c0 = 0; c0 < chunks; c0 += 64 * U)
            __syncthreads();
        return;
    }
    // B rows past N are read from the last row (their sums are not stored)
    const uint8_t *brow[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        brow[r] = B + (int64_t)min(n0 + r, N - 1) * rowBytes;

    int acc[MR][R];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[m][r] = 0;

    // the output this lane writes (see the reduction below) and its scale,
    // loaded first: its latency overlaps the stream's
    const int myV = lane >> (6 - kLogV);  // sum index m * R + r held at the end
    const int myM = myV / R, myN = n0 + myV % R;
    // (clamped indices, no branch: no wait until the value is used)
    uint16_t scBits = 0, xsBits = 0;
    if constexpr (F16OUT) {
        scBits = scale[min(myN, N - 1)];
        xsBits = (xscale ? xscale : scale)[xscale ? min(myM, M - 1) : 0];
    }
    // A in LDS piece-major: 1 KB block u * kH + h holds the 16-byte piece h
    // of chunks 64 u + i (i = 0 ... 63) at 16 i, so that the 64 lanes' reads
    // of one piece are consecutive 16-byte words (free of bank conflicts; a
    // chunk-major layout puts the lanes 32 or 64 bytes apart).  The DMA lane
    // i of block (u, h) reads that piece of chunk 64 u + i; the pass's offset
    // goes in the scalar operand.
    constexpr int kH = kAPerChunk / 16;  // 16-byte pieces of A per chunk
    uint32_t dmaOff[kAPass / 1024];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < kH; ++h)
            dmaOff[u * kH + h] = (uint32_t)(64 * u + lane) * kAPerChunk + 16u * h;

    for (int c0 = 0, pass = 0; c0 < chunks; c0 += 64 * U, ++pass) {
        uint8_t(*as)[kAPass] = As[pass & 1];
        // A of this pass into LDS: wavefront 0, 1 KB DMA blocks (k past K
        // reads as zeros); issued before its B loads, so that its wait for
        // the B loads' count leaves only them in flight
        if (wave == 0) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < M) {
                    const v4si ra = make_rsrc(A + (int64_t)m * K, (uint32_t)K);
#pragma unroll
                    for (int d = 0; d < kAPass / 1024; ++d)
                        dma16(ra, lds_addr(&as[m][1024 * d]), dmaOff[d], (uint32_t)(c0 * kAPerChunk));
                }
            }
        }
        // B: every lane issues all its loads (clamped addresses, so the
        // count is fixed)
        uint4 b[R][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = min(c0 + lane + 64 * u, chunks - 1);
#pragma unroll
            for (int r = 0; r < R; ++r)
                b[r][u] = *(const uint4 *)(brow[r] + (int64_t)c * 16);
        }
        if (wave == 0)
            wait_vmcnt<R * U>();  // the A DMA has landed
        __syncthreads();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // chunks past the row: A reads as zero there (the DMA's range), so
            // the clamped B chunk adds nothing
            uint4 a[MR][kAPerChunk / 16];
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int h = 0; h < kH; ++h)
                    a[m][h] = m < M ? *(const uint4 *)&as[m][1024 * (u * kH + h) + 16 * lane]
                                    : make_uint4(0, 0, 0, 0);
            // the A bytes of the chunk in the order the packed B bytes unpack
            // in (once per chunk, shared by the wavefront's R rows)
            uint32_t ap[MR][kAPerChunk / 4];
#pragma unroll
            for (int m = 0; m < MR; ++m)
                order_a<BITS>(a[m], ap[m]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t o[kAPerChunk / 4];
                unpack_b<BITS>(b[r][u], o);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    // two independent chains of dot products
                    int s0 = acc[m][r], s1 = 0;
#pragma unroll
                    for (int i = 0; i < kAPerChunk / 4; i += 2) {
                        s0 = __builtin_amdgcn_sdot4((int)ap[m][i], (int)o[i], s0, false);
                        s1 = __builtin_amdgcn_sdot4((int)ap[m][i + 1], (int)o[i + 1], s1, false);
                    }
                    acc[m][r] = s0 + s1;
                }
            }
        }
    }

    // ---- reduction: kV sums per lane -> one full sum per lane ----
    // At the step with partner offset o (32, 16, ...) while more than one sum
    // is held, a lane keeps the upper half of its sums if its lane bit o is
    // set, else the lower half, and adds its partner's copy of that half;
    // after log2(kV) steps lane l holds (a partial of) sum l >> (6 - log2 kV).
    // The remaining offsets 32 and 16 are plain butterfly steps; the sum over
    // the 16 lanes of a row (offsets 8 ... 1) uses DPP lane permutes when
    // those offsets are not needed for halving.
    int v[kV];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
            v[m * R + r] = acc[m][r];
#pragma unroll
    for (int st = 0; st < kLogV; ++st) {
        const int o = 32 >> st;
        const int cnt = kV >> st;
        const bool up = (lane & o) != 0;
#pragma unroll
        for (int j = 0; j < cnt / 2; ++j) {
            const int send = up ? v[j] : v[j + cnt / 2];
            const int keep = up ? v[j + cnt / 2] : v[j];
            v[j] = keep + __shfl_xor(send, o, 64);
        }
    }
    int sum = v[0];
    if constexpr (kLogV <= 2) {
#pragma unroll
        for (int o = 32 >> kLogV; o >= 16; o >>= 1)
            sum += __shfl_xor(sum, o, 64);
        sum = row_sum16(sum);
    } else {
#pragma unroll
        for (int o = 32 >> kLogV; o > 0; o >>= 1)
            sum += __shfl_xor(sum, o, 64);
    }

    // the first lane holding each sum writes it
    if ((lane & ((64 >> kLogV) - 1)) == 0 && myM < M && myN < N) {
        const int x = sum >> Up::kShift;  // exact: a multiple of 2^kShift
        if (F16OUT) {
            float sc = __half2float(__ushort_as_half(scBits));
            if (xscale)
                sc *= __half2float(__ushort_as_half(xsBits));  // exact in fp32
            ((__half *)C)[(int64_t)myM * N + myN] = __float2half_rn(apply_act((float)x * sc, act));
        }
        else
            ((int *)C)[(int64_t)myM * N + myN] = x;
    }
}

template <int BITS, int MR, int R, int WAVES, int U>
hipError_t launch_t(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                    void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    const int64_t wgs = ((int64_t)N + R * WAVES - 1) / (R * WAVES);
    if (!grid_fits(wgs, 64 * WAVES))
        return kGridTooLarge;
    const dim3 grid((unsigned)wgs, (unsigned)batch);
    if (scale)
        gemv_kernel<BITS, MR, R, WAVES, U, true><<<grid, 64 * WAVES, 0, s>>>(A, B, scale, xscale, act, C, M, N, K, bs);
    else
        gemv_kernel<BITS, MR, R, WAVES, U, false><<<grid, 64 * WAVES, 0, s>>>(A, B, scale, xscale, act, C, M, N, K, bs);
    return hipGetLastError();
}


// Wavefront shapes: (rows of B per wavefront, wavefronts per workgroup).
template <int BITS, int MR>
hipError_t launch_cfg(int idx, const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale,
                      int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    // a lane's chunks per row per pass: 64 * U chunks cover K = 4096
    constexpr int U = BITS == 8 ? 4 : BITS == 4 ? 2 : 1;
    switch (idx) {
    case 0: return launch_t<BITS, MR, 1, 8, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 1: return launch_t<BITS, MR, 1, 16, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 2: return launch_t<BITS, MR, 2, 4, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    default: return launch_t<BITS, MR, 2, 8, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    }
}

// Measured on MI355X (kernel trace, K = 4096, each launch on a different B
// past the caches; shapes 1x8, 1x16, 2x4, 2x8, 4x2, 4x4, 4x8 and 8x4 tried):
//   int2: two rows, eight wavefronts (M = 1: 3.48 us at N = 4096, 5.00 at
//         11008; M = 4: 5.38 / 9.38);
//   int4: up to 6144 rows one row, sixteen wavefronts (M = 1: 3.76 us at
//         N = 4096, the time of a plain read of the same 8.4 MB); above
//         that two rows, eight wavefronts (6.12 at N = 11008), four for
//         M >= 3 (10.70 against 11.02);
//   int8: one row; sixteen wavefronts up to 6144 rows for M <= 2 (4.68 us),
//         else eight (8.98 at N = 11008); two rows, four wavefronts for
//         M >= 3 above 6144 rows (11.90).
// Four or eight rows per wavefront were slower at M > 1 in every case.
int choose_cfg(int M, int N, int bits, int batch)
{
    const bool small = (int64_t)N * batch <= 6144;
    if (bits == 2)
        return 3;
    if (bits == 4)
        return small ? 1 : M >= 3 ? 2 : 3;
    if (small)
        return M <= 2 ? 1 : 0;
    return M <= 2 ? 0 : 2;
}

template <int BITS>
hipError_t launch_m(int idx, const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale,
                    int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    if (M == 1)
        return launch_cfg<BITS, 1>(idx, A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    if (M == 2)
        return launch_cfg<BITS, 2>(idx, A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    return launch_cfg<BITS, 4>(idx, A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
}

}  // namespace

hipError_t launch_gemv(const int8_t *A, const uint8_t *B, int bits, const uint16_t *scale,
                       const uint16_t *xscale, int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs,
                       hipStream_t s)
{
    if (M == 0 || N == 0)
        return hipSuccess;
    const int idx = choose_cfg(M, N, bits, batch);
    switch (bits) {
    case 8: return launch_m<8>(idx, A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 4: return launch_m<4>(idx, A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    default: return launch_m<2>(idx, A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    }
}

}  // namespace bq
