// Streaming GEMM for skinny M (decode / small batch): M <= 64.
//
// Computes acc[m,n] = sum_k A[m,k] * B[n,k] (BitBLAS custom-operator guide,
// section 1 and case 1) and optionally C = fp16(acc * scale[n]) (section 2).
// At M <= 64 the arithmetic intensity is below the MI355X ridge point, so
// the kernel is built to stream B from HBM exactly once at full bandwidth:
//
//  * B goes straight from global memory into matrix-core operand registers
//    (no LDS): lane l of a wavefront owns row n = n0 + (l & 15) of B and the
//    32-byte piece (l >> 4) of each 128-byte segment of that row; four lanes
//    cover a 128-byte line per row per iteration.
//  * int4 / int2 bytes are unpacked in registers (unpack.h) into signed int8
//    operands, so the matrix cores consume them as int8.
//  * v_mfma_i32_16x16x64_i8: the A operand is the (zero-padded) 16-row tile
//    of A, the B operand the 16 rows of B; a lane's operand bytes cover the
//    same 16 consecutive k in both (row/column = lane & 15, k group =
//    lane >> 4), so the k order inside an instruction is irrelevant to the
//    integer sum.  M = 1 wastes 15/16 of the matrix-core work, which is
//    still far below the time to stream B.
//  * A workgroup of four wavefronts splits the K range of its column block
//    four ways; each wavefront issues the loads of a whole group of
//    iterations before using them, and the four partial int32 tiles are
//    summed through LDS before the epilogue (exact: integer addition).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "unpack.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
constexpr int kSegBytes = 128;  // bytes of one B row consumed per iteration
constexpr int kGroup = 4;       // iterations whose loads are issued together

__device__ __forceinline__ uint4 load16(const uint8_t *p) { return load_nt16(p); }

template <int BITS, int MT, int NT, bool F16OUT>
__global__ __launch_bounds__(kThreads) void gemm_stream_kernel(
    const int8_t *__restrict__ A, const uint8_t *__restrict__ B,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ xscale, int act,
    void *__restrict__ C,
    int M, int N, int K, BatchStrides bs)
{
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
    using U = Unpack<BITS>;
    constexpr int kValsPerLane = 32 * 8 / BITS;    // k values in a lane's 32 bytes
    constexpr int kMfmaPerIt = kValsPerLane / 16;  // 16 k per operand
    constexpr int kSpan = 4 * kValsPerLane;        // k covered per iteration

    __shared__ int red[4][MT][NT][256];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;  // A row / B row within a 16-tile
    const int lg = lane >> 4;  // k group
    const int n0 = blockIdx.x * (16 * NT);

    const int64_t rowBytes = (int64_t)K * BITS / 8;
    const int iters = (int)((rowBytes + kSegBytes - 1) / kSegBytes);
    const int itBeg = (iters * wave) / 4;
    const int itEnd = (iters * (wave + 1)) / 4;

    const uint8_t *brow[NT];
    bool bvalid[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + nt * 16 + li;
        bvalid[nt] = n < N;
        brow[nt] = B + (int64_t)(bvalid[nt] ? n : 0) * rowBytes;
    }
    const int8_t *arow[MT];
    bool avalid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + li;
        avalid[mt] = m < M;
        arow[mt] = A + (int64_t)(avalid[mt] ? m : 0) * K;
    }

    v4i acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = (v4i){0, 0, 0, 0};

    for (int itg = itBeg; itg < itEnd; itg += kGroup) {
        uint4 braw[kGroup][NT][2];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const int64_t off = (int64_t)(itg + u) * kSegBytes + lg * 32;
            const bool itok = (itg + u) < itEnd;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool ok = itok && bvalid[nt] && (off + 16 * h) < rowBytes;
                    braw[u][nt][h] = ok ? load16(brow[nt] + off + 16 * h) : make_uint4(0, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            if ((itg + u) >= itEnd)
                break;
            const int kbase = (itg + u) * kSpan + lg * kValsPerLane;
            uint32_t bop[NT][2 * U::kOutDwords];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                U::run(braw[u][nt][0], &bop[nt][0]);
                U::run(braw[u][nt][1], &bop[nt][U::kOutDwords]);
            }
#pragma unroll
            for (int t = 0; t < kMfmaPerIt; ++t) {
                const int k = kbase + t * 16;
                v4i a[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    // Zero operand for padded rows and for k past the end (K % 64
                    // == 0, so a 16-byte piece is wholly inside or outside).
                    a[mt] = (avalid[mt] && k < K) ? *(const v4i *)(arow[mt] + k) : (v4i){0, 0, 0, 0};
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const v4i b = {(int)bop[nt][4 * t + 0], (int)bop[nt][4 * t + 1],
                                   (int)bop[nt][4 * t + 2], (int)bop[nt][4 * t + 3]};
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt], b, acc[mt][nt], 0, 0, 0);
                }
            }
        }
    }

    // Output tile layout of the 16x16 instruction: lane l holds column l & 15
    // and rows 4*(l >> 4) + r, r = 0..3.  Store as [row][col] in LDS.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][mt][nt][(4 * lg + r) * 16 + li] = acc[mt][nt][r];
    __syncthreads();

    const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + row;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = n0 + nt * 16 + col;
            const int e = row * 16 + col;
            int v = red[0][mt][nt][e] + red[1][mt][nt][e] + red[2][mt][nt][e] + red[3][mt][nt][e];
            v >>= U::kShift;  // exact: the sum is a multiple of 2^kShift
            if (m < M && n < N) {
                if (F16OUT) {
                    // weight scale, times the row's activation scale when given
                    // (a product of two fp16 values: exact in fp32)
                    float s = __half2float(__ushort_as_half(scale[n]));
                    if (xscale)
                        s *= __half2float(__ushort_as_half(xscale[m]));
                    ((__half *)C)[(int64_t)m * N + n] = __float2half_rn(apply_act((float)v * s, act));
                } else {
                    ((int *)C)[(int64_t)m * N + n] = v;
                }
            }
        }
    }
}

template <int BITS, int MT, int NT>
hipError_t launch_t(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                    void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    const dim3 grid((unsigned)((N + 16 * NT - 1) / (16 * NT)), (unsigned)batch);
    if (scale)
        gemm_stream_kernel<BITS, MT, NT, true><<<grid, kThreads, 0, s>>>(A, B, scale, xscale, act, C, M, N, K, bs);
    else
        gemm_stream_kernel<BITS, MT, NT, false><<<grid, kThreads, 0, s>>>(A, B, scale, xscale, act, C, M, N, K, bs);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                       void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    if (M <= 16)
        return launch_t<BITS, 1, 1>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    if (M <= 32)
        return launch_t<BITS, 2, 2>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    return launch_t<BITS, 4, 2>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
}

}  // namespace

hipError_t launch_gemm_stream(const int8_t *A, const uint8_t *B, int bits,
                              const uint16_t *scale, const uint16_t *xscale, int act, void *C,
                              int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    if (M == 0 || N == 0)
        return hipSuccess;
    switch (bits) {
    case 8: return launch_bits<8>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 4: return launch_bits<4>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    default: return launch_bits<2>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    }
}

}  // namespace bq
