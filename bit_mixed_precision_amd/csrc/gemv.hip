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
//  * every load of a lane (its chunks of all R rows, and the bytes of A
//    they multiply, which are the same for every row and are loaded once) is
//    issued before any is used, and the weight scale of the output the lane
//    writes just before them, so no memory latency follows the stream;
//  * packed values are unpacked in registers to 16 v / 64 v bytes (unpack.h)
//    and multiplied with v_dot4_i32_i8;
//  * the R x MR lane sums are reduced across the wavefront by a butterfly that
//    halves the number of values at each of the first log2(R MR) steps (each
//    lane keeps the half its partner does not, and adds the partner's copy of
//    it), so R MR sums cost R MR - 1 + 6 - log2(R MR) exchanges instead of
//    6 R MR, those within a 16-lane row as DPP operands of the adds; the
//    lane that ends with sum (m, r) writes that output.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
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
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = (blockIdx.x * WAVES + wave) * R;
    if (n0 >= N)
        return;
    const int64_t rowBytes = (int64_t)K * BITS / 8;
    const int chunks = (int)(rowBytes / 16);  // K % 64 == 0: whole chunks
    const uint8_t *brow = B + (int64_t)n0 * rowBytes;

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
    float sc = 1.0f;
    if (F16OUT && myM < M && myN < N) {
        sc = __half2float(__ushort_as_half(scale[myN]));
        if (xscale)
            sc *= __half2float(__ushort_as_half(xscale[myM]));  // exact in fp32
    }

    for (int c0 = 0; c0 < chunks; c0 += 64 * U) {
        uint4 b[R][U];
        uint4 a[MR][U][kAPerChunk / 16];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            const bool ok = c < chunks;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bool rok = ok && (n0 + r) < N;
                b[r][u] = rok ? load_nt16(brow + (int64_t)r * rowBytes + (int64_t)c * 16) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            const bool ok = c < chunks;
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
            for (int r = 0; r < R; ++r) {
                uint32_t o[Up::kOutDwords];
                Up::run(b[r][u], o);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    // two independent chains of dot products
                    int s0 = acc[m][r], s1 = 0;
#pragma unroll
                    for (int h = 0; h < kAPerChunk / 16; ++h) {
                        s0 = __builtin_amdgcn_sdot4((int)a[m][u][h].x, (int)o[4 * h + 0], s0, false);
                        s1 = __builtin_amdgcn_sdot4((int)a[m][u][h].y, (int)o[4 * h + 1], s1, false);
                        s0 = __builtin_amdgcn_sdot4((int)a[m][u][h].z, (int)o[4 * h + 2], s0, false);
                        s1 = __builtin_amdgcn_sdot4((int)a[m][u][h].w, (int)o[4 * h + 3], s1, false);
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
        if (F16OUT)
            ((__half *)C)[(int64_t)myM * N + myN] = __float2half_rn(apply_act((float)x * sc, act));
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
    case 0: return launch_t<BITS, MR, 1, 4, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 1: return launch_t<BITS, MR, 2, 4, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 2: return launch_t<BITS, MR, 4, 4, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 3: return launch_t<BITS, MR, 8, 4, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 4: return launch_t<BITS, MR, 2, 8, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 5: return launch_t<BITS, MR, 4, 8, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 6: return launch_t<BITS, MR, 4, 2, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    default: return launch_t<BITS, MR, 8, 2, U>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    }
}

// Measured on MI355X (kernel trace, K = 4096, each launch on a different B
// past the caches): at M = 1 one row per wavefront up to 6144 rows per
// launch (int4 N = 4096: 4.48 us against 4.54 / 4.56 for two / four rows),
// four rows above that (int4 N = 11008: 6.84 against 7.60 with one; int8
// two: 9.58 against 9.66); at M = 2 two rows (4.84 / 7.70 us for int4).
int choose_cfg(int M, int N, int bits, int batch)
{
    const int64_t rows = (int64_t)N * batch;
    if (M == 1) {
        if (rows <= 6144)
            return 0;
        return bits == 8 ? 1 : 2;
    }
    return 1;
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
