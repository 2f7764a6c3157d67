// Decode GEMV for the W4A16 GEMM with NF4 weight codes (M <= 4): fp16 A
// [M, K], NF4 codes B [N, K/2] (two per byte, low nibble = even k),
// per-row scale and zero point; C = fp16(sum_k A[m,k] W[n,k]) with
// W[n,k] = fp16((table[c] - zero[n]) * scale[n]) computed in fp32 and the
// sum accumulated in fp32 (BitBLAS custom-operator guide, case 2).
//
// Like the integer GEMV, this is a stream over B (four bits per weight):
//  * one wavefront per ROWS (1 or 2) rows of B; its lanes walk the packed
//    row in 16-byte chunks (32 codes), lane l taking chunks l, l + 64, ...;
//    all of a lane's chunk loads of a batch are issued before any is used;
//  * each wavefront first builds, for each of its rows, a 256-entry table in
//    LDS mapping a packed byte (two codes) to the two dequantized fp16
//    weights, so one 4-byte LDS read decodes two weights;
//  * v_dot2_f32_f16 multiplies pairs of fp16 activations and weights into
//    fp32 lane sums, reduced across the wavefront with butterfly shuffles.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "nf4_table.h"

namespace bq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_sum_f(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Dequantized weight of code c for the row with scale s and zero point z:
// fp16(fp32(table[c] - z) * s), two fp32 roundings then one to fp16.  The
// empty asm makes the fp32 product a value of its own, so the compiler cannot
// fuse the multiply with the conversion (a mixed-precision FMA, which would
// round the exact product to fp16 once).
__device__ __forceinline__ uint32_t nf4_weight(int c, float s, float z)
{
    const float d = __half2float(__ushort_as_half(kNf4TableF16[c])) - z;
    float w = d * s;
    asm volatile("" : "+v"(w));
    return __half_as_ushort(__float2half_rn(w));
}

// MR rows of A, ROWS rows of B per wavefront, U chunks per lane per batch.
template <int MR, int ROWS, int U>
__global__ __launch_bounds__(kThreads) void gemv_nf4_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ B, const uint16_t *__restrict__ scale,
    const uint16_t *__restrict__ zero, uint16_t *__restrict__ C, int M, int N, int K)
{
    __shared__ uint32_t lut[kWaves][ROWS][256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = (blockIdx.x * kWaves + wave) * ROWS;
    if (n0 >= N)
        return;

    // byte -> (weight of the low-nibble code, weight of the high-nibble code)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int n = min(n0 + r, N - 1);  // a row past N gets a valid table; its result is not written
        const float s = __half2float(__ushort_as_half(scale[n]));
        const float z = zero ? __half2float(__ushort_as_half(zero[n])) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = lane + 64 * i;
            lut[wave][r][b] = nf4_weight(b & 15, s, z) | (nf4_weight(b >> 4, s, z) << 16);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int64_t rowBytes = K / 2;
    const int chunks = (int)(rowBytes / 16);  // K % 64 == 0: whole chunks

    float acc[MR][ROWS];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            acc[m][r] = 0.0f;

    for (int c0 = 0; c0 < chunks; c0 += 64 * U) {
        uint4 b[ROWS][U];
        uint4 a[MR][U][4];  // 32 fp16 activations per chunk
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
                for (int h = 0; h < 4; ++h)
                    a[m][u][h] = (ok && m < M) ? *(const uint4 *)(A + (int64_t)m * K + (int64_t)c * 32 + 8 * h)
                                               : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                // 16 packed bytes -> 16 pairs of fp16 weights (k = 2i, 2i+1)
                const uint32_t pw[4] = {b[r][u].x, b[r][u].y, b[r][u].z, b[r][u].w};
                uint32_t w[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    w[i] = lut[wave][r][(pw[i >> 2] >> (8 * (i & 3))) & 0xFFu];
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    float s = acc[m][r];
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t av[4] = {a[m][u][h].x, a[m][u][h].y, a[m][u][h].z, a[m][u][h].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, av[e]),
                                                       __builtin_bit_cast(h2, w[4 * h + e]), s, false);
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
            acc[m][r] = wave_sum_f(acc[m][r]);

    // lane (m * ROWS + r) writes output (m, n0 + r)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int n = n0 + r;
            if (lane == m * ROWS + r && m < M && n < N)
                C[(int64_t)m * N + n] = __half_as_ushort(__float2half_rn(acc[m][r]));
        }
}

template <int MR, int kRows>
hipError_t launch_t(const uint16_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *zero, uint16_t *C,
                    int M, int N, int K, hipStream_t s)
{
    // kRows rows x 2 chunks of 16 bytes per lane per batch: one batch covers K = 4096
    constexpr int kU = 2;
    const int64_t wgs = ((int64_t)N + kRows * kWaves - 1) / (kRows * kWaves);
    if (!grid_fits(wgs, kThreads))
        return kGridTooLarge;
    const dim3 grid((unsigned)wgs);
    gemv_nf4_kernel<MR, kRows, kU><<<grid, kThreads, 0, s>>>(A, B, scale, zero, C, M, N, K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_nf4(const uint16_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *zero,
                           uint16_t *C, int M, int N, int K, hipStream_t s)
{
    if (M == 0 || N == 0)
        return hipSuccess;
    // M = 1: one B row per wavefront up to N = 6144, two above (as for the
    // integer GEMV; back to back at K = 4096: N = 4096 5.38 against 5.64 us,
    // N = 11008 11.3 against 9.6 us)
    if (M == 1)
        return N <= 6144 ? launch_t<1, 1>(A, B, scale, zero, C, M, N, K, s)
                         : launch_t<1, 2>(A, B, scale, zero, C, M, N, K, s);
    if (M == 2)
        return launch_t<2, 2>(A, B, scale, zero, C, M, N, K, s);
    return launch_t<4, 2>(A, B, scale, zero, C, M, N, K, s);
}

}  // namespace bq
