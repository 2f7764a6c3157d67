// Streaming matrix-core GEMM for small and mid-sized M (3 <= M <= 256):
// acc[m,n] = sum_k A[m,k] * B[n,k] in int32 (BitBLAS custom-operator guide,
// section 1 and case 1), optionally C = fp16(acc * scale[n]) (section 2).
//
// Below the MI355X ridge point (about 625 int8 operations per byte) the
// GEMM is bound by moving operands, not by the matrix cores.  With a few
// hundred output tiles of TM x TN, each CU has to bring in its tile's rows of
// A (from L2, shared by every tile of those rows) and of B (from HBM, read
// once in all): (TM + TN * bits/8) * K bytes.  The kernel is built so that
// this traffic is nearly all it does:
//
//  * The wavefronts of a workgroup split K (Pallas matmul page, blocked
//    matmul: the K blocks of one output block are independent partial sums):
//    K is cut in chunks of 128, wavefront w takes chunks w, w + WK, ...,
//    and keeps the next two of its chunks in flight.  No wavefront waits for
//    another inside the K loop.
//  * Each chunk's rows of A and packed B go from global memory to the
//    wavefront's own LDS buffers with the LDS-DMA form of the 16-byte buffer
//    load, 1 KB of consecutive row bytes per instruction (loads into
//    matrix-core operand layout directly would put 16 rows in each 16-lane
//    group and cost the address unit one cache line per cycle instead of one
//    4-lane quad); rows past M / N and k past K read as zeros.  The rows are
//    XOR-swizzled at 16-byte granularity so that the operand reads are free
//    of bank conflicts.
//  * Operands are read from LDS into the v_mfma_i32_16x16x64_i8 layout;
//    int4 / int2 are unpacked in registers (unpack.h), so every packed B byte
//    is loaded and unpacked once per workgroup.  Inside a chunk a lane owns
//    32 consecutive k of its row (lane group g = lane / 16 takes k [32 g,
//    32 g + 32)) and at sub-step s feeds k [32 g + 16 s, +16) of both
//    operands; the instruction sums over whatever k its lanes feed, so the
//    integer sum is the full dot product.
//  * The WK partial tiles are summed through LDS (exact: integer addition),
//    lane-major so that the LDS accesses are conflict-free, and the epilogue
//    (weight scale, optional token scale and activation, one rounding to
//    fp16) runs on the sums.  No partial sum leaves the workgroup.
//  * Tiles are ordered so that the workgroups one XCD runs (blockIdx modulo
//    8 picks the XCD) share their B rows: a B tile is read from HBM into one
//    XCD's L2 and used there by every M tile.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "lds_dma.h"
#include "unpack.h"

namespace bq {
namespace {

constexpr int kXcds = 8;
constexpr int kKC = 128;  // k per chunk

// Compiler and instruction-scheduler fence: no memory operation or
// instruction is moved across it.
__device__ __forceinline__ void fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Chunk layout of one operand in LDS: rows of P bytes (the chunk's 128 k at
// BITS bits), 16-byte pieces XOR-swizzled by a function of the row bits
// above the rows that share a 256-byte bank line.  A ds_read_b128 is served
// 16 lanes per cycle from 64 four-byte banks, the lanes of one cycle being
// those with equal lane bit 5 and equal parity of lane bits 2..4; the
// fragment reads below take row 16 f + (lane & 15) and piece lane >> 4 (or
// 2 (lane >> 4) + s), and with s = row / kL, s ^ (s << 1) puts the 16 lanes
// of each cycle in 16 distinct bank groups (the plain s puts them two to a
// group).
template <int P>
struct Rows {
    static constexpr int kQ = P / 16;          // 16-byte pieces per row
    static constexpr int kL = 256 / P;         // rows per 256-byte bank line
    static constexpr int kPerKB = 1024 / P;    // rows per 1 KB DMA instruction
    __device__ __forceinline__ static int phys(int row, int piece)
    {
        const int s = row / kL;
        return piece ^ ((s ^ (s << 1)) & (kQ - 1));
    }
};

// TM x TN output tile per workgroup; WN wavefronts split the tile's columns
// (TN / WN each), WK wavefronts split K.  F16OUT: fp16 epilogue.
template <int BITS, int TM, int TN, int WN, int WK, bool F16OUT>
__global__ __launch_bounds__(64 * WN * WK) void gemm_stream_kernel(
    const int8_t *__restrict__ A, const uint8_t *__restrict__ B,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ xscale, int act,
    void *__restrict__ C, int M, int N, int K, int tilesM, int tilesN, BatchStrides bs)
{
    constexpr int kTNW = TN / WN;                 // columns per wavefront
    constexpr int FM = TM / 16, FN = kTNW / 16;   // 16 x 16 fragments per wavefront
    constexpr int kF = FM * FN;
    static_assert(TM % 16 == 0 && kTNW % 16 == 0 && TN % WN == 0, "tile shape");
    using U = Unpack<BITS>;
    using RA = Rows<kKC>;
    using RB = Rows<kKC * BITS / 8>;
    constexpr int kPB = kKC * BITS / 8;           // packed B bytes per row per chunk
    constexpr int kSA = TM * kKC, kSB = kTNW * kPB;
    constexpr int kBuf = kSA + kSB;               // one chunk of one wavefront
    constexpr int kDmaA = kSA / 1024;
    constexpr int kDmaB = (kSB + 1023) / 1024;
    constexpr int kLanesLastB = (kSB - 1024 * (kDmaB - 1)) / 16;  // active lanes of the last B DMA
    constexpr int kDma = kDmaA + kDmaB;           // DMA instructions per chunk
    static_assert(kSA % 1024 == 0 && kSB % 256 == 0 && kDma < 32, "chunk shape");
    static_assert(kF * 4 * 64 * 4 <= 2 * kBuf, "partial sums fit in a wavefront's buffers");

    __shared__ __attribute__((aligned(1024))) int8_t lds[WN * WK * 2 * kBuf];

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

    // ---- tile coordinates: the tiles of one XCD are consecutive in M-fastest
    // order, so the M tiles of a B column block share that XCD's L2 ----
    const int total = tilesM * tilesN;
    int t = blockIdx.x;
    if (total % kXcds == 0)
        t = (t % kXcds) * (total / kXcds) + t / kXcds;
    const int tm = t % tilesM, tn = t / tilesM;
    const int m0 = tm * TM;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wk = wave % WK, wn = wave / WK;
    const int nw0 = tn * TN + wn * kTNW;          // first B row of this wavefront
    const int li = lane & 15, lg = lane >> 4;

    const uint32_t rowB = (uint32_t)K * BITS / 8;  // packed bytes per B row
    const v4si rA = make_rsrc(A + (int64_t)m0 * K, (uint32_t)(min(M - m0, TM) * K));
    const v4si rB = make_rsrc(B + (int64_t)nw0 * rowB, nw0 < N ? (uint32_t)min(N - nw0, kTNW) * rowB : 0u);
    int8_t *const wl = lds + wave * 2 * kBuf;     // this wavefront's two chunk buffers
    const uint32_t wlAddr = lds_addr(wl);

    // ---- scales of the outputs this wavefront finishes (fragments f = wk,
    // wk + WK, ... of its column block), loaded before the stream with
    // clamped indices (no branch, so no wait until they are used) ----
    constexpr int kMineF = (kF + WK - 1) / WK;
    uint16_t scBits[kMineF], xsBits[kMineF][4];
    const uint16_t *xsp = xscale ? xscale : scale;
    const int xsLim = xscale ? M - 1 : 0;
#pragma unroll
    for (int u = 0; u < kMineF; ++u) {
        const int f = min(wk + u * WK, kF - 1);
        const int i = f / FN, j = f % FN;
        if constexpr (F16OUT) {
            scBits[u] = scale[min(nw0 + 16 * j + li, N - 1)];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                xsBits[u][r] = xsp[min(m0 + 16 * i + 4 * lg + r, xsLim)];
        }
    }
    fence();

    // ---- per-lane DMA source offsets within a chunk (chunk k offset added
    // per load); the lane's 16 bytes land at LDS row r, piece phys(r, lc) ----
    uint32_t aOff[kDmaA], bOff[kDmaB];
    int aK[kDmaA], bK[kDmaB];  // first k of the lane's 16 bytes within the chunk
#pragma unroll
    for (int d = 0; d < kDmaA; ++d) {
        const int r = d * RA::kPerKB + lane / RA::kQ, pc = lane % RA::kQ;
        const int lc = RA::phys(r, pc);  // the swizzle is its own inverse
        aOff[d] = (uint32_t)r * (uint32_t)K + 16u * lc;
        aK[d] = 16 * lc;
    }
#pragma unroll
    for (int d = 0; d < kDmaB; ++d) {
        const int r = d * RB::kPerKB + lane / RB::kQ, pc = lane % RB::kQ;
        const int lc = RB::phys(r, pc);
        bOff[d] = (uint32_t)r * rowB + 16u * lc;
        bK[d] = 16 * lc * 8 / BITS;
    }
    const int nch = (K + kKC - 1) / kKC;
    // For int8 B the chunk order is rotated by the tile's column block, so
    // that the workgroups streaming different B rows at the same time are at
    // different k, while the M tiles of one column block stay together and
    // share B in their XCD's L2 (W8A8 M = 64, N = 12288: 16.5 -> 15.2 us with
    // 64 x 64 tiles, 14.5 -> 13.6 with 64 x 48).  For int4 / int2 B at
    // N = K = 4096 the rotation cost 1-6 %, so they keep the plain order.  The
    // sums do not depend on the order.
    const int rot = (BITS == 8 && nch > 0) ? (tn * 3) % nch : 0;
    // DMA of chunk c into buffer b (zeros for k past K: each 16 bytes of a
    // row is wholly below or above K, a multiple of 64)
    auto issue = [&](int c, int b) {
        const uint32_t base = wlAddr + b * kBuf;
        const int k0 = (c + rot < nch ? c + rot : c + rot - nch) * kKC;
#pragma unroll
        for (int d = 0; d < kDmaA; ++d)
            dma16(rA, base + 1024 * d, k0 + aK[d] < K ? aOff[d] + (uint32_t)k0 : kOOB, 0);
#pragma unroll
        for (int d = 0; d < kDmaB; ++d) {
            const uint32_t off = k0 + bK[d] < K ? bOff[d] + (uint32_t)(k0 * BITS / 8) : kOOB;
            if (d < kDmaB - 1 || kLanesLastB == 64 || lane < kLanesLastB)
                dma16(rB, base + kSA + 1024 * d, off, 0);
        }
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = (v4i){0, 0, 0, 0};

    // operands of one chunk from buffer b into the matrix-core layout, and
    // the matrix work on them (two sub-steps of 64 k)
    auto compute = [&](int b) {
        const int8_t *la = wl + b * kBuf;
        const int8_t *lb = la + kSA;
        v4i a[FM][2], bo[FN][2];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = 16 * i + li;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                a[i][s] = *(const v4i *)(la + r * kKC + 16 * RA::phys(r, 2 * lg + s));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int r = 16 * j + li;
            if constexpr (BITS == 8) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    bo[j][s] = *(const v4i *)(lb + r * kPB + 16 * RB::phys(r, 2 * lg + s));
            } else if constexpr (BITS == 4) {
                // the lane's 32 k are 16 packed bytes: k 0-15 in dwords x, y
                const uint4 p = *(const uint4 *)(lb + r * kPB + 16 * RB::phys(r, lg));
                bo[j][0] = U::template operand<0>(p);
                bo[j][1] = U::template operand<1>(p);
            } else {
                // 8 packed bytes: k 0-15 in the first dword
                const uint2 p = *(const uint2 *)(lb + r * kPB + 16 * RB::phys(r, lg >> 1) + 8 * (lg & 1));
                uint32_t o0, o1, o2, o3;
                unpack16_int2(p.x, o0, o1, o2, o3);
                bo[j][0] = (v4i){(int)o0, (int)o1, (int)o2, (int)o3};
                unpack16_int2(p.y, o0, o1, o2, o3);
                bo[j][1] = (v4i){(int)o0, (int)o1, (int)o2, (int)o3};
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i][s], bo[j][s], acc[i][j], 0, 0, 0);
    };

    // ---- this wavefront's chunks wk, wk + WK, ...; two in flight ----
    const int mine = nch > wk ? (nch - wk + WK - 1) / WK : 0;
    if (mine > 0)
        issue(wk, 0);
    if (mine > 1)
        issue(wk + WK, 1);
    for (int q = 0; q < mine; ++q) {
        // chunk q has landed (only chunk q + 1's loads may still be in flight)
        if (q + 1 < mine)
            wait_vmcnt<kDma>();
        else
            wait_vmcnt<0>();
        fence();
        compute(q & 1);
        // the buffer's reads completed before the matrix work that used them;
        // only then is it refilled
        fence();
        if (q + 2 < mine)
            issue(wk + (q + 2) * WK, q & 1);
    }

    // ---- sum of the WK partial tiles: each wavefront's sums go into its own
    // (now idle) buffers, lane-major ----
    {
        int *red = (int *)wl;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[((i * FN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < kMineF; ++u) {
        const int f = wk + u * WK;
        if (f >= kF)
            break;
        const int i = f / FN, j = f % FN;
        const int n = nw0 + 16 * j + li;
        int v[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < WK; ++w) {
            const int *red = (const int *)(lds + (wn * WK + w) * 2 * kBuf);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] += red[(f * 4 + r) * 64 + lane];
        }
        // output layout of the 16 x 16 instruction: lane l holds column
        // l & 15 and rows 4 (l >> 4) + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 16 * i + 4 * lg + r;
            if (m < M && n < N) {
                if constexpr (F16OUT) {
                    // scale / 2^kShift folds the exact int4 / int2 rescaling
                    // into the multiply; the token scale is a product of two
                    // fp16 values, exact in fp32
                    float sc = __half2float(__ushort_as_half(scBits[u])) * (1.0f / (float)(1 << U::kShift));
                    if (xscale)
                        sc *= __half2float(__ushort_as_half(xsBits[u][r]));
                    const float y = apply_act((float)v[r] * sc, act);
                    ((__half *)C)[(int64_t)m * N + n] = __float2half_rn(y);
                } else {
                    ((int *)C)[(int64_t)m * N + n] = v[r] >> U::kShift;  // exact
                }
            }
        }
    }
}

template <int BITS, int TM, int TN, int WN, int WK>
hipError_t launch_t(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                    void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    const int64_t tilesM = (M + TM - 1) / TM, tilesN = (N + TN - 1) / TN;
    if (!grid_fits(tilesM * tilesN, 64 * WN * WK))
        return kGridTooLarge;
    const dim3 grid((unsigned)(tilesM * tilesN), (unsigned)batch);
    if (scale)
        gemm_stream_kernel<BITS, TM, TN, WN, WK, true><<<grid, 64 * WN * WK, 0, s>>>(
            A, B, scale, xscale, act, C, M, N, K, (int)tilesM, (int)tilesN, bs);
    else
        gemm_stream_kernel<BITS, TM, TN, WN, WK, false><<<grid, 64 * WN * WK, 0, s>>>(
            A, B, scale, xscale, act, C, M, N, K, (int)tilesM, (int)tilesN, bs);
    return hipGetLastError();
}


// Wavefronts splitting K for a tile: eight while their chunk buffers (two
// chunks each) fit in 128 KB of LDS, else four.
constexpr int stream_wk(int bits, int tm, int tn)
{
    return 2 * 8 * (tm * kKC + tn * kKC * bits / 8) <= 128 * 1024 ? 8 : 4;
}

// Tile configurations (TM x TN, one column of wavefronts).
struct Cfg {
    int tm, tn;
};
constexpr Cfg kCfgs[] = {{16, 16}, {16, 32}, {16, 64}, {32, 32}, {32, 64}, {64, 32}, {64, 48}, {64, 64}};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BITS, int C>
hipError_t launch_c(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                    void *C_, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    constexpr int TM = kCfgs[C].tm, TN = kCfgs[C].tn;
    return launch_t<BITS, TM, TN, 1, stream_wk(BITS, TM, TN)>(A, B, scale, xscale, act, C_, M, N, K, batch, bs, s);
}

template <int BITS>
hipError_t launch_cfg(int idx, const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale,
                      int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    switch (idx) {
    case 0: return launch_c<BITS, 0>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 1: return launch_c<BITS, 1>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 2: return launch_c<BITS, 2>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 3: return launch_c<BITS, 3>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 4: return launch_c<BITS, 4>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 5: return launch_c<BITS, 5>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    case 6: return launch_c<BITS, 6>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    default: return launch_c<BITS, 7>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
    }
}

// The configuration for a shape, by a traffic model (checked against every
// configuration at N = K = 4096, M = 8 ... 256, and W8A8 M = 64, N = 12288:
// it picks the fastest or one within 1 %): with T tiles of TM x TN
// on 256 CUs the busiest CU moves ceil(T / 256) (TM + TN bits/8) K operand
// bytes at the per-CU rate (about 75 GB/s measured, LDS-DMA into a
// workgroup's buffers), while B, N K bits/8 bytes, leaves HBM once (about
// 5.5 TB/s); the estimate is the larger of the two, the two rates entering
// as their ratio, with padded outputs as a tie-break, then the squarer tile
// (32 x 32 over 16 x 64: 6.1 against 6.5 us at M = 64, N = K = 4096, int4
// and int2).  When the winner runs in one round of workgroups, a tiling of
// the same height that ties with it and keeps more CUs busy in one round
// is taken instead (W8A8 M = 64, N = 12288: 64 x 48 on all 256 CUs 14.5 us,
// 64 x 64 on 192 CUs 15.7 us; both bound by the same HBM bytes).
int choose_cfg(int M, int N, int bits, int batch)
{
    constexpr int64_t kCUs = 256;
    constexpr int64_t kHbmOverCu = 73;  // HBM rate / per-CU operand rate (5.5 TB/s / 75 GB/s)
    int64_t main[kNumCfgs], tiles[kNumCfgs];
    int best = 0;
    int64_t bestCost = INT64_MAX;
    for (int c = 0; c < kNumCfgs; ++c) {
        const Cfg &g = kCfgs[c];
        tiles[c] = (int64_t)((M + g.tm - 1) / g.tm) * ((N + g.tn - 1) / g.tn) * batch;
        const int64_t rounds = (tiles[c] + kCUs - 1) / kCUs;
        // per-K byte counts, times 8 to keep the int2 quarter byte integral
        const int64_t perCu = rounds * (8 * g.tm + g.tn * bits);
        const int64_t hbm = (int64_t)N * bits * batch / kHbmOverCu;
        const int64_t waste = tiles[c] * g.tm * g.tn - (int64_t)M * N * batch;  // padded outputs
        main[c] = (perCu > hbm ? perCu : hbm) * 64 + waste / 64;
        const int64_t skew = g.tm > g.tn ? g.tm - g.tn : g.tn - g.tm;
        const int64_t cost = main[c] * 64 + skew;
        if (cost < bestCost) {
            bestCost = cost;
            best = c;
        }
    }
    if (tiles[best] <= kCUs) {
        int pick = best;
        for (int c = 0; c < kNumCfgs; ++c)
            if (kCfgs[c].tm == kCfgs[best].tm && main[c] == main[best] && tiles[c] <= kCUs &&
                tiles[c] > tiles[pick])
                pick = c;
        best = pick;
    }
    return best;
}

template <int BITS>
hipError_t launch_bits(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale, int act,
                       void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s)
{
    return launch_cfg<BITS>(choose_cfg(M, N, BITS, batch), A, B, scale, xscale, act, C, M, N, K, batch, bs, s);
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
