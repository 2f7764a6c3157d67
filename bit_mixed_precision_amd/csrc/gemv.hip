// Decode GEMV (M <= 4): acc[m,n] = sum_k A[m,k] * B[n,k], optionally
// C = fp16(acc * scale[n]) (BitBLAS custom-operator guide, sections 1-2 and
// case 1).
//
// At M <= 4 every byte of B is used by at most 4 multiply-adds, so the kernel
// is a stream over B and its speed is set by how fast B leaves HBM.  It is
// laid out like a plain streaming read:
//  * one wavefront per ROWS (1 or 2) rows of B; its 64 lanes walk the
//    packed row in 16-byte chunks (lane l takes chunks l, l+64, ...), so one
//    load instruction covers 1 KB of a row;
//  * all of a lane's chunk loads (for every row) are issued before any is
//    used; the matching bytes of A (at most 4 rows, a few KB) come from the
//    L1/L2 caches, fetched in the same batch;
//  * the packed values are unpacked in registers to 16*v / 64*v bytes
//    (unpack.h) and multiplied with v_dot4_i32_i8; the lane partial sums are
//    reduced across the wavefront with butterfly shuffles;
//  * many small workgroups (four wavefronts each) keep every CU busy.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "unpack.h"

namespace bq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// MR rows of A, ROWS rows of B per wavefront, U chunks per lane per batch.
template <int BITS, int MR, int ROWS, int U, bool F16OUT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
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
    using Up = Unpack<BITS>;
    constexpr int kAPerChunk = 16 * 8 / BITS;  // bytes of A (= k values) per packed chunk
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = (blockIdx.x * kWaves + wave) * ROWS;
    if (n0 >= N)
        return;
    const int64_t rowBytes = (int64_t)K * BITS / 8;
    const int chunks = (int)(rowBytes / 16);  // K % 64 == 0: whole chunks

    int acc[MR][ROWS];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            acc[m][r] = 0;

    for (int c0 = 0; c0 < chunks; c0 += 64 * U) {
        uint4 b[ROWS][U];
        uint4 a[MR][U][kAPerChunk / 16];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            const bool ok = c < chunks;
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const bool rok = ok && (n0 + r) < N;
                b[r][u] = rok ? load_nt16(B + (int64_t)(n0 + r) * rowBytes + (int64_t)c * 16)
                              : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int h = 0; h < kAPerChunk / 16; ++h)
                    a[m][u][h] = (ok && m < M) ? *(const uint4 *)(A + (int64_t)m * K + (int64_t)c * kAPerChunk + 16 * h)
                                               : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                uint32_t o[Up::kOutDwords];
                Up::run(b[r][u], o);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    int s = acc[m][r];
#pragma unroll
                    for (int h = 0; h < kAPerChunk / 16; ++h) {
                        s = __builtin_amdgcn_sdot4((int)a[m][u][h].x, (int)o[4 * h + 0], s, false);
                        s = __builtin_amdgcn_sdot4((int)a[m][u][h].y, (int)o[4 * h + 1], s, false);
                        s = __builtin_amdgcn_sdot4((int)a[m][u][h].z, (int)o[4 * h + 2], s, false);
                        s = __builtin_amdgcn_sdot4((int)a[m][u][h].w, (int)o[4 * h + 3], s, false);
                    }
                    acc[m][r] = s;
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            acc[m][r] = wave_sum(acc[m][r]);

    // lane (m * ROWS + r) writes output (m, n0 + r)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int n = n0 + r;
            if (lane == m * ROWS + r && m < M && n < N) {
                const int v = acc[m][r] >> Up::kShift;  // exact: a multiple of 2^kShift
                if (F16OUT) {
                    // weight scale, times the row's activation scale when given
                    // (a product of two fp16 values: exact in fp32)
                    float sc = __half2float(__ushort_as_half(scale[n]));
                    if (xscale)
                        sc *= __half2float(__ushort_as_half(xscale[m]));
                    ((__half *)C)[(int64_t)m * N + n] = __float2half_rn(apply_act((float)v * sc, act));
                } else
                    ((int *)C)[(int64_t)m * N + n] = v;
            }
        }
}

template <int BITS, int MR, int ROWS, int U>
hipError_t launch_t(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                    void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    const int waves = (N + ROWS - 1) / ROWS;
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves), (unsigned)batch);
    if (scale)
        gemv_kernel<BITS, MR, ROWS, U, true><<<grid, kThreads, 0, s>>>(A, B, scale, xscale, act, C, M, N, K, bs);
    else
        gemv_kernel<BITS, MR, ROWS, U, false><<<grid, kThreads, 0, s>>>(A, B, scale, xscale, act, C, M, N, K, bs);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                       void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    // a lane's loads per batch: ROWS rows x U chunks of B (64 B of packed B
    // per row at U = 4 / 2 / 1 for 8 / 4 / 2 bits: one batch covers K = 4096)
    constexpr int U = BITS == 8 ? 4 : BITS == 4 ? 2 : 1;
    // M = 1: one B row per wavefront for int8 at any N and for int4 / int2
    // up to 6144 rows in all (more, smaller wavefronts start streaming
    // sooner), two above that (fewer wavefronts to launch).  Measured back to
    // back at K = 4096: int4 N = 4096 3.94 against 4.17 us, N = 11008 7.2
    // against 6.4 us; int8 one row is ahead at every N from 1024 to 14336.
    if (M == 1) {
        if (BITS == 8 || (int64_t)N * batch <= 6144)
            return launch_t<BITS, 1, 1, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
        return launch_t<BITS, 1, 2, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    }
    if (M == 2)
        return launch_t<BITS, 2, 2, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    return launch_t<BITS, 4, 2, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
}

}  // namespace

hipError_t launch_gemv(const int8_t *A, const uint8_t *B, int bits, const uint16_t *scale,
                       const uint16_t *xscale, int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
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
