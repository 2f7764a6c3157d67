// LDS-tiled matrix-core GEMM for prefill-sized M.
//
// Computes acc[m,n] = sum_k A[m,k] * B[n,k] (BitBLAS custom-operator guide,
// section 1 and case 1) with an int32 accumulator that stays in registers
// for the whole K loop, and converts once at the end (the Pallas matmul
// page's pattern: a wide accumulator, one downcast after the last K block),
// optionally to C = fp16(acc * scale[n]) (BitBLAS guide, section 2).
//
// Decomposition (Pallas page, blocked matmul: output blocks independent,
// the K blocks accumulated in sequence): a workgroup of four wavefronts owns
// a BM x BN output tile and walks K in 128-byte steps.  Per step:
//  * A (int8) and B (int8, or packed int4/int2 unpacked in registers on the
//    way in, see unpack.h) are loaded from global memory with 16-byte loads
//    and written to LDS as [row][128] int8 with the 16-byte chunk index
//    XOR-swizzled by the row, so that the matrix-core operand reads of 32
//    consecutive rows at one k offset spread over all banks;
//  * LDS is double buffered: the global loads for step s+1 are issued before
//    the matrix-core work of step s and stored after it; one barrier per
//    step;
//  * each wavefront computes a (BM/2) x (BN/2) quadrant with
//    v_mfma_i32_32x32x32_i8 (the A operand gives 32 rows of A, the B operand
//    32 rows of B; each lane's 16 operand bytes are 16 consecutive k, the
//    same k for both operands).
// Workgroups are mapped so that the tiles one XCD runs (blockIdx modulo 8
// picks the XCD) form a compact block of the output, sharing A and B rows in
// that XCD's L2.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "unpack.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;  // unpacked k per step = bytes per LDS row
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int BITS, int BM, int BN, bool F16OUT>
__global__ __launch_bounds__(kThreads) void gemm_tiled_kernel(
    const int8_t *__restrict__ A, const uint8_t *__restrict__ B,
    const uint16_t *__restrict__ scale, void *__restrict__ C, int M, int N, int K,
    int tilesM, int tilesN)
{
    using U = Unpack<BITS>;
    constexpr int kPB = kBK * BITS / 8;          // packed B bytes per row per step
    constexpr int kCPR = kPB / 16;               // packed 16-byte chunks per row
    constexpr int kBRowsPerPass = kThreads / kCPR;
    constexpr int kBPasses = BN / kBRowsPerPass;
    constexpr int kAPasses = BM / 32;            // A: 8 chunks per row, 32 rows per pass
    constexpr int kUnpackChunks = 8 / BITS;      // LDS chunks produced per packed chunk
    constexpr int kFM = BM / 64;                 // 32x32 fragments per wave, M
    constexpr int kFN = BN / 64;                 // and N
    static_assert(kBPasses >= 1 && BN % kBRowsPerPass == 0, "tile/pass mismatch");

    __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * kBK];

    // ---- tile coordinates (XCD-aware) ----
    const int total = tilesM * tilesN;
    int t = blockIdx.x;
    if (total % kXcds == 0)
        t = (t % kXcds) * (total / kXcds) + t / kXcds;
    const int perGroup = kGroupM * tilesN;
    const int group = t / perGroup;
    const int firstM = group * kGroupM;
    const int gsz = min(tilesM - firstM, kGroupM);
    const int tm = firstM + (t % perGroup) % gsz;
    const int tn = (t % perGroup) / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int64_t rowBytesB = (int64_t)K * BITS / 8;
    const int steps = (K + kBK - 1) / kBK;

    // ---- global -> register staging ----
    const int aChunk = tid & 7, aRow = tid >> 3;
    const int bChunk = tid % kCPR, bRow = tid / kCPR;
    uint4 ra[kAPasses], rb[kBPasses];

    auto gload = [&](int step) {
        const int k0 = step * kBK;
#pragma unroll
        for (int p = 0; p < kAPasses; ++p) {
            const int m = m0 + p * 32 + aRow;
            const int k = k0 + aChunk * 16;
            ra[p] = (m < M && k < K) ? *(const uint4 *)(A + (int64_t)m * K + k) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < kBPasses; ++p) {
            const int n = n0 + p * kBRowsPerPass + bRow;
            const int64_t off = (int64_t)step * kPB + bChunk * 16;
            rb[p] = (n < N && off < rowBytesB) ? *(const uint4 *)(B + (int64_t)n * rowBytesB + off)
                                               : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
        int8_t *la = lds[buf];
        int8_t *lb = lds[buf] + BM * kBK;
#pragma unroll
        for (int p = 0; p < kAPasses; ++p) {
            const int row = p * 32 + aRow;
            *(uint4 *)(la + row * kBK + swz(row, aChunk) * 16) = ra[p];
        }
#pragma unroll
        for (int p = 0; p < kBPasses; ++p) {
            const int row = p * kBRowsPerPass + bRow;
            uint32_t o[U::kOutDwords];
            U::run(rb[p], o);
#pragma unroll
            for (int u = 0; u < kUnpackChunks; ++u) {
                const int chunk = bChunk * kUnpackChunks + u;
                *(uint4 *)(lb + row * kBK + swz(row, chunk) * 16) =
                    make_uint4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3]);
            }
        }
    };

    v16i acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j)
            acc[i][j] = (v16i){};

    gload(0);
    sstore(0);
    __syncthreads();

    const int fr = lane & 31;  // operand row within a 32-row fragment
    const int fg = lane >> 5;  // k half (16 bytes) within a 32-k sub-step
    for (int step = 0; step < steps; ++step) {
        const int buf = step & 1;
        if (step + 1 < steps)
            gload(step + 1);
        const int8_t *la = lds[buf];
        const int8_t *lb = lds[buf] + BM * kBK;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int chunk = ks * 2 + fg;
            v4i a[kFM], b[kFN];
#pragma unroll
            for (int i = 0; i < kFM; ++i) {
                const int row = wm * (BM / 2) + i * 32 + fr;
                a[i] = *(const v4i *)(la + row * kBK + swz(row, chunk) * 16);
            }
#pragma unroll
            for (int j = 0; j < kFN; ++j) {
                const int row = wn * (BN / 2) + j * 32 + fr;
                b[j] = *(const v4i *)(lb + row * kBK + swz(row, chunk) * 16);
            }
#pragma unroll
            for (int i = 0; i < kFM; ++i)
#pragma unroll
                for (int j = 0; j < kFN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (step + 1 < steps)
            sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    // 32x32 output layout: lane l holds column l & 31; register r holds row
    // 8*(r/4) + 4*(l >> 5) + (r & 3).
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
        const int n = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
        float s = 0.f;
        if (F16OUT && n < N)
            s = __half2float(__ushort_as_half(scale[n]));
#pragma unroll
        for (int i = 0; i < kFM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) {
                    const int v = acc[i][j][r] >> U::kShift;
                    if (F16OUT)
                        ((__half *)C)[(int64_t)m * N + n] = __float2half_rn((float)v * s);
                    else
                        ((int *)C)[(int64_t)m * N + n] = v;
                }
            }
        }
    }
}

template <int BITS, int BM, int BN>
hipError_t launch_t(const int8_t *A, const uint8_t *B, const uint16_t *scale, void *C,
                    int M, int N, int K, hipStream_t s)
{
    const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tilesM * tilesN));
    if (scale)
        gemm_tiled_kernel<BITS, BM, BN, true><<<grid, kThreads, 0, s>>>(A, B, scale, C, M, N, K, tilesM, tilesN);
    else
        gemm_tiled_kernel<BITS, BM, BN, false><<<grid, kThreads, 0, s>>>(A, B, scale, C, M, N, K, tilesM, tilesN);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const int8_t *A, const uint8_t *B, const uint16_t *scale, void *C,
                       int M, int N, int K, hipStream_t s)
{
    // 256x256 tiles once there are enough of them to fill the 256 CUs.
    const int64_t tiles256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    if (tiles256 >= 256)
        return launch_t<BITS, 256, 256>(A, B, scale, C, M, N, K, s);
    return launch_t<BITS, 128, 128>(A, B, scale, C, M, N, K, s);
}

}  // namespace

hipError_t launch_gemm_tiled(const int8_t *A, const uint8_t *B, int bits,
                             const uint16_t *scale, void *C, int M, int N, int K,
                             hipStream_t s)
{
    if (M == 0 || N == 0)
        return hipSuccess;
    switch (bits) {
    case 8: return launch_bits<8>(A, B, scale, C, M, N, K, s);
    case 4: return launch_bits<4>(A, B, scale, C, M, N, K, s);
    default: return launch_bits<2>(A, B, scale, C, M, N, K, s);
    }
}

}  // namespace bq
