// LDS-tiled matrix-core GEMM for prefill-sized M.
//
// Computes acc[m,n] = sum_k A[m,k] * B[n,k] (BitBLAS custom-operator guide,
// section 1 and case 1) with an int32 accumulator that stays in registers
// for the whole K loop, and converts once at the end (the Pallas matmul
// page's pattern: a wide accumulator, one downcast after the last K block),
// optionally to C = fp16(acc * scale[n]) (BitBLAS guide, section 2).
//
// Decomposition (Pallas page, blocked matmul: output blocks independent, the
// K blocks accumulated in sequence): a workgroup owns a BM x BN output tile
// (256 x 256, 128 x 128 or 64 x 64, with two to eight wavefronts; chosen by
// the number of tiles and the width of B, see launch_bits) and walks K in
// stages of 128.
//
//  * Global -> LDS without registers: 16-byte buffer loads with the LDS-DMA
//    form (lane i of a load writes LDS bytes [M0 + 16 i, +16)).  Rows past
//    M / N and k past K are outside the buffer range and arrive as zeros.
//    B stays packed in LDS (int4: 64 bytes per row per stage, int2: 32).
//    The 1 KB blocks of a stage are dealt round-robin to the wavefronts.
//  * A ring of STAGES LDS buffers; the loads of stage s+STAGES-1 are issued
//    while stage s is computed, so HBM/L2 latency is covered by whole stages.
//  * Every LDS row is XOR-swizzled at 16-byte granularity so that the 16
//    lanes served together by a 16-byte operand read hit 16 distinct 16-byte
//    bank groups (rows of 128 / 64 / 32 bytes use the row bits above the
//    2 / 4 / 8 rows that share one 256-byte bank line).  The load lanes are
//    permuted so that the DMA writes exactly this layout.
//  * Wavefronts form a 2 x (WAVES/2) grid over the tile (1 x WAVES for
//    some configurations, so that one wavefront unpacks each B column) and
//    compute with v_mfma_i32_32x32x32_i8, A fragments as the first operand
//    and B fragments as the second (each lane owns 4 consecutive rows m of
//    one column n).  Under a sustained matrix-core load the clock is set by
//    power, and this operand order draws less of it than the reverse with
//    int8 activations against shifted int4 / int2 weights: M = N = K = 4096
//    runs 4% (W4A8) and 7% (W2A8) faster, W8A8 and the fp16 NF4 mode the
//    same.  Per 32-k sub-step a lane feeds 16 consecutive k of each
//    operand; packed B is read 16 bytes at a time and unpacked in registers
//    (unpack.h) into 1, 2 or 4 sub-steps.  The 256 x 256 int4 ping-pong
//    loop uses v_mfma_i32_16x16x64_i8 instead (16 x 16 fragments, two 64-k
//    sub-steps per stage), which holds a higher clock for the same work.
//  * Wave tiles of several fragments read the fragments of sub-step j+1
//    while the matrix cores run j, with one barrier per stage placed between
//    the two halves of the last sub-step.  32 x 32 wave tiles (one matrix
//    instruction per sub-step) instead read a whole stage of operands one
//    stage ahead.
//  * Epilogue: fp16(acc * scale) values are staged through LDS (neighbouring
//    lanes trade halves so that each LDS write holds two adjacent columns)
//    and written as 16-byte coalesced streaming (nontemporal) stores.
//  * With few output tiles and a workspace from the caller, K is split over
//    several workgroups per tile; the last to finish adds the others'
//    partial sums (SplitK below).
//  * An NF4 mode (fp16 activations, 4-bit NormalFloat weight codes) reuses
//    the same ring and loops with fp16 matrix-core operands (see the kernel).
// Workgroups are mapped so that the tiles one XCD runs (blockIdx modulo 8
// picks the XCD) form a compact block of the output, sharing A and B rows in
// that XCD's L2.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "lds_dma.h"
#include "nf4_decode.h"
#include "unpack.h"

namespace bq {
namespace {

constexpr int kBK = 128;  // unpacked k per stage
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// 16-byte chunk permutation of an LDS row (XOR with a function of the row):
// the DMA stores logical chunk c of row r at physical chunk c ^ swz(r), the
// fragment reads undo it.  A ds_read_b128 is served 16 lanes per cycle from
// 64 four-byte banks, the 16 lanes of one cycle being those with equal lane
// bit 5 and equal parity of lane bits 2..4 (measured with bank-conflict
// counters on lane pairs).  With s = the row's bits from `shift` up, the
// plain s spreads the reads of 32-row fragments over all 64 banks in each
// cycle, but puts the 16-row fragment reads of the 16x16x64 loop two to a
// bank; s ^ (s << 1) (GRAY) serves both conflict-free.
template <bool GRAY>
__device__ __forceinline__ int swz(int row, int shift, int mask)
{
    const int s = row >> shift;
    return (GRAY ? s ^ (s << 1) : s) & mask;
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// One matrix-core step on a 32 x 32 tile: int8 x int8 -> int32 over 32 k,
// or (NF4) fp16 x fp16 -> fp32 over 16 k; A fragment first.
template <bool NF4, typename Acc>
__device__ __forceinline__ Acc mma32(const v4i &a, const v4i &b, const Acc &c)
{
    if constexpr (NF4)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Bit pattern of one accumulator element (taken by value: a bit cast of a
// vector element in place is not reliable).
__device__ __forceinline__ uint32_t bits32(int x) { return (uint32_t)x; }
__device__ __forceinline__ uint32_t bits32(float x) { return __float_as_uint(x); }

__device__ __forceinline__ uint32_t dword_of(const uint4 &p, int i)
{
    return i == 0 ? p.x : i == 1 ? p.y : i == 2 ? p.z : p.w;
}

// K split of each output tile over `parts` workgroups: workgroup q of a tile
// runs the 128-k stages [q stepsPer, (q+1) stepsPer) and stores its int32
// partial sums; the last of the tile's workgroups to arrive (a per-tile
// counter) adds the others' partial sums to its own and runs the epilogue.
// Integer addition is exact, so the result does not depend on the split.
struct SplitK {
    int parts = 1;           // workgroups per output tile
    int stepsPer = 0;        // 128-k stages per workgroup
    int *ctr = nullptr;      // per-tile arrival counters, zero between launches
    int4 *part = nullptr;    // partial sums: [tile][part][16-byte piece][thread]
};

// WGM: wavefronts along M (2, or 1 for a 1 x WAVES grid whose wave tiles
// span all BM rows, so that each B column is decoded by one wavefront).
template <int BITS, int BM, int BN, int STAGES, bool F16OUT, int WAVES, bool NF4 = false, int WGM = 2>
struct TiledCfg {
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kWGN = WAVES / WGM;            // wave grid: WGM along M, WAVES/WGM along N
    static constexpr int kPB = kBK * BITS / 8;          // packed B bytes per row per stage
    static constexpr int kCPR = kPB / 16;               // B 16-byte chunks per row
    static constexpr int kRowsPerLineB = 256 / kPB;     // B rows sharing a 256-byte bank line
    static constexpr int kSwzShiftB = ilog2(kRowsPerLineB);
    // A rows use the GRAY chunk permutation on the 256 x 256 tiles: there it
    // removes the 16x16x64 loop's bank conflicts (M = N = K = 4096 W4A8 3-6 %
    // faster) and, on the 32 x 32 loops, measured no slower with the same
    // (zero) conflicts (W2A8 and NF4 2-4 % faster, W8A8 even); on the
    // 128 x 128 W4A8 tile it measured 4-5 % slower at M = 1024 in four runs,
    // so the smaller tiles keep the plain one.  B rows keep the plain one:
    // GRAY measured no faster on any tile, the ping-pong loop's included.
    static constexpr bool kGrayA = BM == 256 && BN == 256;
    static constexpr int kSA = BM * kBK;                // A bytes per stage
    static constexpr int kSB = BN * kPB;                // B bytes per stage
    static constexpr int kStage = kSA + kSB;
    // 1 KB DMA blocks per stage, dealt round-robin to the wavefronts (block b
    // to wave b % WAVES); when a count is not a multiple of WAVES the last
    // round leaves some waves without a block
    static constexpr int kBlkA = kSA / 1024;
    static constexpr int kBlkB = kSB / 1024;
    static constexpr int kDmaA = (kBlkA + WAVES - 1) / WAVES;  // block rounds per stage
    static constexpr int kDmaB = (kBlkB + WAVES - 1) / WAVES;
    static constexpr bool kEvenA = kBlkA % WAVES == 0, kEvenB = kBlkB % WAVES == 0;
    static constexpr int kDma = kDmaA + kDmaB;          // DMA instructions per stage, upper bound per wave
    static constexpr int kWM = BM / WGM, kWN = BN / kWGN; // wave tile
    static constexpr int kFM = kWM / 32;                // 32x32 fragments per wave along M
    static constexpr int kFN = kWN / 32;                // and N
    static constexpr int kSPR = 8 / BITS;               // sub-steps fed by one packed 16-byte read
    // epilogue staging: 64 rows (or fewer) of kWN outputs (fp16 or int32) per
    // wave, rows padded by 32 bytes (bank offsets of the staging writes and
    // copy-out reads below)
    static constexpr int kES = F16OUT ? 2 : 4;          // bytes per output element
    static constexpr int kEpiPitch = kWN * kES + 32;
    // 64 rows per pass, or 32 where 64 rows of every wave's tile would not fit in LDS
    static constexpr int kEpiRows = kWM < 64 ? kWM : WAVES * 64 * kEpiPitch <= 160 * 1024 ? 64 : 32;
    static constexpr int kEpiBytes = WAVES * kEpiRows * kEpiPitch;
    static constexpr int kRing = STAGES * kStage;
    static constexpr int kLds = (kRing > kEpiBytes) ? kRing : kEpiBytes;
    static_assert(kSA % 1024 == 0 && kSB % 1024 == 0, "whole 1 KB DMA blocks");
    static_assert(kLds <= 160 * 1024, "LDS");
    // 32 x 32 wave tiles read their operands a whole stage ahead instead of
    // one sub-step ahead: a single matrix instruction per sub-step cannot
    // cover the LDS latency.
    static constexpr bool kAhead = kFM * kFN == 1;
    static_assert(!kAhead || STAGES >= 4, "stage-ahead loop keeps STAGES-3 stages of loads in flight");
    static_assert(kFN >= 1 && kFM >= 1 && (kFM == 1 || kFM % 2 == 0), "wave tile");
};

// FUSE: fp16 epilogue with the optional per-row activation scale (xscale,
// NULL meaning 1) and the activation act; the plain fp16 epilogue has none.
// SPLIT: the K split above (blockIdx.x = part * tiles + tile).
// NF4: fp16 activations and 4-bit NF4 weight codes (BitBLAS custom-operator
// guide, case 2).  A is fp16 [M, K/2] in the kernel's byte terms: K here is
// the byte width of an A row (twice the number of k), so a stage of 128 A
// bytes is 64 k, and the packed B row (K/4 bytes in these terms, two codes
// per byte) has the int2 layout (BITS = 2).  `scale` is the per-row weight
// scale and `xscale` the per-row zero point (NULL = 0): every lane first
// builds the dequantized 16-entry table of each B row it feeds in registers,
// fp16((table[c] - zero) * scale) in fp32; the matrix cores then take fp16
// operands (v_mfma_f32_32x32x16_f16) and the fp32 sums go out as fp16.
template <int BITS, int BM, int BN, int STAGES, bool F16OUT, bool KTAIL, int WAVES, bool FUSE, bool SPLIT,
          bool NF4 = false, int WGM = 2>
__global__ __launch_bounds__(64 * WAVES) void gemm_tiled_kernel(
    const int8_t *__restrict__ A, const uint8_t *__restrict__ B,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ xscale, int act, void *__restrict__ C,
    int M, int N, int K, int tilesM, int tilesN, BatchStrides bs, SplitK sk)
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
    using T = TiledCfg<BITS, BM, BN, STAGES, F16OUT, WAVES, NF4, WGM>;
    // the ping-pong loop below: eight wavefronts (two per SIMD) in a 2 x 4
    // grid over a 256 x 256 tile of int4 B, three LDS stages.  Measured on
    // MI355X at M = N = 4096 (kernel trace, against the loop further down):
    // K = 4096 60.6 against 61.1 us, K = 8192 107.5 against 111.2 us; for
    // int2 B it gained nothing at K = 4096 and lost 4 us at K = 1024.
    constexpr bool kPP = BM == 256 && BN == 256 && WAVES == 8 && WGM == 2 && STAGES == 3 && !NF4 && !SPLIT &&
                         BITS == 4;
    // The ping-pong loop runs v_mfma_i32_16x16x64_i8 (16 x 16 output
    // fragments), every other loop v_mfma_i32_32x32x32_i8 (32 x 32): under a
    // sustained load the matrix cores hold a higher clock with the smaller
    // instruction for the same work (a loop of the W4A8 GEMM's operands:
    // 4.3-4.4 against 3.9 POP/s).
    constexpr bool kM16 = kPP;
    constexpr int kCF = kM16 ? 16 : 32;                      // output fragment edge
    constexpr int kFMe = T::kWM / kCF, kFNe = T::kWN / kCF;  // fragments per wavefront
    static_assert(!NF4 || (BITS == 2 && F16OUT && !FUSE), "NF4: int2 byte layout, fp16 output, no fused epilogue");
    constexpr int kThreads = T::kThreads;
    static_assert(STAGES >= 2 && STAGES <= 8, "two to eight LDS stages");
    static_assert((STAGES - 2) * T::kDma < 64, "outstanding loads fit the wait counter");

    __shared__ __attribute__((aligned(1024))) int8_t lds[T::kLds];

    // ---- tile coordinates (XCD-aware) ----
    const int total = tilesM * tilesN;
    int t = blockIdx.x;
    int split = 0;
    if constexpr (SPLIT) {
        split = t / total;
        t -= split * total;
    }
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
    // the wavefront index is uniform: keep it (and every LDS address derived
    // from it) in scalar registers
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::kWGN, wn = wave % T::kWGN;

    const uint32_t rowBytesB = (uint32_t)((int64_t)K * BITS / 8);
    // this workgroup's 128-k stages: [s0, s0 + steps) of the whole K
    const int s0 = SPLIT ? split * sk.stepsPer : 0;
    const int steps = SPLIT ? min((K + kBK - 1) / kBK - s0, sk.stepsPer) : (K + kBK - 1) / kBK;

    // Buffer resources over this tile's rows: rows past M / N are past the end.
    const v4si srcA = make_rsrc(A + (int64_t)m0 * K, (uint32_t)(min(M - m0, BM) * K));
    const v4si srcB = make_rsrc(B + (int64_t)n0 * rowBytesB, (uint32_t)min(N - n0, BN) * rowBytesB);
    const uint32_t ldsBase = (uint32_t)(uintptr_t)(lds_void_t *)lds;

    // ---- DMA address setup: lane -> (row, logical chunk) of each 1 KB block ----
    // A block b (rows 8b..8b+7): lane s -> row 8b + s/8, physical chunk s%8.
    const int aRowInBlk = lane >> 3;
    uint32_t aOff[T::kDmaA];
    int aChunkL[T::kDmaA];
#pragma unroll
    for (int p = 0; p < T::kDmaA; ++p) {
        const int row = (wave + WAVES * p) * 8 + aRowInBlk;
        aChunkL[p] = (lane & 7) ^ swz<T::kGrayA>(row, 1, 7);
        aOff[p] = (uint32_t)row * (uint32_t)K + aChunkL[p] * 16;
    }
    // B block b (1024 / kPB rows): lane s -> row (1024/kPB) b + s / kCPR, chunk s % kCPR.
    constexpr int kBRowsPerBlk = 1024 / T::kPB;
    uint32_t bOff[T::kDmaB];
    int bChunkL[T::kDmaB];
#pragma unroll
    for (int p = 0; p < T::kDmaB; ++p) {
        const int row = (wave + WAVES * p) * kBRowsPerBlk + lane / T::kCPR;
        bChunkL[p] = (lane % T::kCPR) ^ swz<false>(row, T::kSwzShiftB, T::kCPR - 1);
        bOff[p] = (uint32_t)row * rowBytesB + bChunkL[p] * 16;
    }

    // This wavefront's DMA instructions per stage (wave-uniform).
    int myDma = 0;
#pragma unroll
    for (int p = 0; p < T::kDmaA; ++p)
        myDma += (wave + WAVES * p < T::kBlkA) ? 1 : 0;
#pragma unroll
    for (int p = 0; p < T::kDmaB; ++p)
        myDma += (wave + WAVES * p < T::kBlkB) ? 1 : 0;
    // Wait until the stage after the current one has landed: with an S-stage
    // ring the loads of S-2 later stages (myDma each) may still be in flight.
    auto wait_stage = [&]() {
        if constexpr (T::kEvenA && T::kEvenB)
            wait_vmcnt<(STAGES - 2) * T::kDma>();
        else
            wait_vmcnt_rt<STAGES - 2, T::kDma>(myDma);
    };

    // Loads of one stage.  Without a K tail (K % 128 == 0) the per-lane
    // offsets are loop invariant and the stage's k offset travels in the
    // scalar soffset; stages past the end re-read the last stage (in range,
    // never consumed).  With a K tail, chunks past K get an out-of-range
    // offset and read as zeros.
    auto issue_stage = [&](int step, int part, int nparts) {
        const uint32_t base = ldsBase + (uint32_t)((step % STAGES) * T::kStage);
        const int sstep = s0 + min(step, steps - 1);
        const int ka = sstep * kBK;
        const uint32_t kb = (uint32_t)sstep * T::kPB;
#pragma unroll
        for (int p = 0; p < T::kDmaA; ++p) {
            if (p % nparts != part || (!T::kEvenA && wave + WAVES * p >= T::kBlkA))
                continue;
            uint32_t voff = aOff[p], soff = (uint32_t)ka;
            if (KTAIL) {
                voff = (ka + aChunkL[p] * 16 < K) ? aOff[p] + (uint32_t)ka : kOOB;
                soff = 0;
            }
            dma16(srcA, base + (wave + WAVES * p) * 1024, voff, soff);
        }
#pragma unroll
        for (int p = 0; p < T::kDmaB; ++p) {
            if ((T::kDmaA + p) % nparts != part || (!T::kEvenB && wave + WAVES * p >= T::kBlkB))
                continue;
            uint32_t voff = bOff[p], soff = kb;
            if (KTAIL) {
                voff = (kb + bChunkL[p] * 16 < rowBytesB) ? bOff[p] + kb : kOOB;
                soff = 0;
            }
            dma16(srcB, base + T::kSA + (wave + WAVES * p) * 1024, voff, soff);
        }
    };

    // ---- LDS -> operand fragments ----
    const int fr = lane & 31;  // row within a 32-row fragment
    const int fg = lane >> 5;  // lane group: which 16 k of a 32-k sub-step
    v4i fa[2][T::kFM];         // A operand fragments, double buffered by sub-step
    uint4 fbp[2][T::kFN];      // packed B, double buffered by packed read
    auto read_a = [&](int step, int ks, int slot) {
        const int8_t *la = lds + (step % STAGES) * T::kStage;
        const int q = ks / T::kSPR, tt = ks % T::kSPR;
        const int chunk = (2 * q + fg) * T::kSPR + tt;
#pragma unroll
        for (int i = 0; i < T::kFM; ++i) {
            const int row = wm * T::kWM + i * 32 + fr;
            fa[slot][i] = *(const v4i *)(la + row * kBK + ((chunk ^ swz<T::kGrayA>(row, 1, 7)) * 16));
        }
    };
    auto read_b = [&](int step, int q, int slot) {
        const int8_t *lb = lds + (step % STAGES) * T::kStage + T::kSA;
        const int chunk = 2 * q + fg;
#pragma unroll
        for (int j = 0; j < T::kFN; ++j) {
            const int row = wn * T::kWN + j * 32 + fr;
            fbp[slot][j] = *(const uint4 *)(lb + row * T::kPB +
                                            ((chunk ^ swz<false>(row, T::kSwzShiftB, T::kCPR - 1)) * 16));
        }
    };

    using Acc = typename std::conditional<NF4, v16f, v16i>::type;
    using AccE = typename std::conditional<kM16, v4i, Acc>::type;
    AccE acc[kFMe][kFNe];
#pragma unroll
    for (int i = 0; i < kFMe; ++i)
#pragma unroll
        for (int j = 0; j < kFNe; ++j)
            acc[i][j] = (AccE){};

    // NF4: the dequantized table of each B row this lane feeds (one per
    // fragment column j), in registers
    Nf4Lut lut[NF4 ? T::kFN : 1];
    if constexpr (NF4) {
#pragma unroll
        for (int j = 0; j < T::kFN; ++j) {
            const int n = n0 + wn * T::kWN + j * 32 + fr;
            // rows past N get zero weights
            lut[j] = n < N ? nf4_lut(scale[n], xscale ? xscale[n] : (uint16_t)0) : Nf4Lut{};
        }
    }

    // B operands of sub-step ks, unpacked from the packed 16-byte read that
    // feeds it (operand tt of that read)
    v4i bop[2][T::kFN];
    auto unpack_b = [&](int ks, int oslot) {
        const int pslot = (ks / T::kSPR) & 1, tt = ks % T::kSPR;
#pragma unroll
        for (int j = 0; j < T::kFN; ++j) {
            const uint4 &pk = fbp[pslot][j];
            if constexpr (NF4)
                bop[oslot][j] = decode_nf4(dword_of(pk, tt), lut[j]);
            else if constexpr (BITS == 8)
                bop[oslot][j] = U::template operand<0>(pk);
            else if constexpr (BITS == 4)
                bop[oslot][j] = tt == 0 ? U::template operand<0>(pk) : U::template operand<1>(pk);
            else
                bop[oslot][j] = tt == 0 ? U::template operand<0>(pk)
                              : tt == 1 ? U::template operand<1>(pk)
                              : tt == 2 ? U::template operand<2>(pk)
                                        : U::template operand<3>(pk);
        }
    };
    // matrix-core work of one sub-step on fragment rows [i0, i1), A-fragment
    // major: each A operand stays in place for kFN consecutive instructions
    // while the B operand changes, an order that draws less power than the
    // reverse (M = N = K = 4096, power-limited: W2A8 3 %, W4A8 0.6 % faster)
    auto mfma_rows = [&](int oslot, int aslot, int i0, int i1) {
        if constexpr (!kM16) {
#pragma unroll
            for (int i = i0; i < i1; ++i)
#pragma unroll
                for (int j = 0; j < T::kFN; ++j)
                    acc[i][j] = mma32<NF4>(fa[aslot][i], bop[oslot][j], acc[i][j]);
        }
    };
    constexpr int kHalf = T::kFM / 2;
    constexpr int kReads = T::kFM + T::kFN;

    // The weight scale of the lane's column in each of its kFN fragments for
    // the fp16 epilogue (fp32, with the exact int4 / int2 rescaling by
    // 2^-kShift folded in), loaded before the K loop so that its latency is
    // hidden by it.
    float sc[(F16OUT && !NF4) ? kFNe : 1];
    if constexpr (F16OUT && !NF4) {
        constexpr float kInv = 1.0f / (float)(1 << U::kShift);
#pragma unroll
        for (int j = 0; j < kFNe; ++j) {
            const int n = n0 + wn * T::kWN + j * kCF + (kM16 ? (lane & 15) : fr);
            sc[j] = n < N ? __half2float(__ushort_as_half(scale[n])) * kInv : 0.0f;
        }
    }

    if constexpr (kPP) {
        // ---- ping-pong loop (256 x 256 tiles of packed B) ----
        // The two wavefronts that share a SIMD (w and w + 4) take turns: while
        // one runs a stage's matrix-core work from registers, the other issues
        // its share of the loads two stages ahead and reads its operands of
        // the stage from LDS.  Each phase ends at a workgroup barrier; group 1
        // (waves 4-7) starts one phase late (an extra barrier at the start,
        // matched by one at the end for group 0), so the groups stay in
        // opposite phases and each SIMD's matrix core always has a wavefront
        // feeding it.
        //
        // Phases are numbered by the barrier that ends them (barrier 0 ends
        // the prologue).  Group 0 reads stage s in phase 2s+1 and computes it
        // in 2s+2; group 1 reads it in 2s+2 and computes it in 2s+3.  Ring
        // buffer (s+2) mod 3 last held stage s-1, read in phases 2s-1 and 2s,
        // so the loads of stage s+2, issued in the reading phase of stage s
        // (2s+1 or 2s+2), never overwrite data still to be read.  Stage s+1 is
        // first read in phase 2s+3, so each wavefront's loads of it must have
        // landed by barrier 2s+2: group 0 waits at the end of its compute
        // phase 2s+2, group 1 at the end of its reading phase 2s+2, both with
        // only their stage s+2 loads still allowed in flight.
        // 16 x 16 x 64 operands: lane l feeds row / column l & 15 of a
        // fragment and, at 64-k sub-step s, the k [32 g + 16 s, +16) of its
        // k group g = l >> 4 in both operands (the instruction sums over
        // whatever k its lanes feed); a lane's 32 k of a stage's B row are
        // one 16-byte packed read, unpacked into the two sub-steps' operands.
        const int grp = wave >> 2;
        const int l16 = lane & 15, g4 = lane >> 4;
        v4i pa[2][kFMe];    // A operands of the stage's two sub-steps
        uint4 pb[kFNe];     // packed B, 32 k per fragment column
        v4i bq[2][kFNe];    // unpacked B operands, double buffered by sub-step
        auto read_all = [&](int step) {
            const int8_t *la = lds + (step % STAGES) * T::kStage;
            const int8_t *lb = la + T::kSA;
#pragma unroll
            for (int j = 0; j < kFNe; ++j) {
                const int row = wn * T::kWN + j * 16 + l16;
                pb[j] = *(const uint4 *)(lb + row * T::kPB + ((g4 ^ swz<false>(row, T::kSwzShiftB, T::kCPR - 1)) * 16));
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int chunk = 2 * g4 + st;
#pragma unroll
                for (int i = 0; i < kFMe; ++i) {
                    const int row = wm * T::kWM + i * 16 + l16;
                    pa[st][i] = *(const v4i *)(la + row * kBK + ((chunk ^ swz<T::kGrayA>(row, 1, 7)) * 16));
                }
            }
        };
        auto unpack_pp = [&](int st, int slot) {
#pragma unroll
            for (int j = 0; j < kFNe; ++j)
                bq[slot][j] = U::operand_rt(pb[j], st);
        };
        // sub-step st's matrix work, A-fragment major (each A operand held
        // for kFNe consecutive instructions)
        auto mma_sub = [&](int st) {
#pragma unroll
            for (int i = 0; i < kFMe; ++i)
#pragma unroll
                for (int j = 0; j < kFNe; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[st][i], bq[st][j], acc[i][j], 0, 0, 0);
        };
        auto barrier = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };
        issue_stage(0, 0, 1);
        issue_stage(1, 0, 1);
        wait_vmcnt<T::kDma>();  // this wavefront's stage 0 loads
        barrier();
        if (grp == 1)
            barrier();
        for (int step = 0; step < steps; ++step) {
            // reading phase
            issue_stage(step + 2, 0, 1);
            read_all(step);
            if (grp == 1)
                wait_vmcnt<T::kDma>();
            wait_lgkmcnt<0>();
            unpack_pp(0, 0);
            barrier();
            // compute phase: sub-step 0 on the matrix cores while the B
            // operands of sub-step 1 are unpacked, then sub-step 1
            mma_sub(0);
            unpack_pp(1, 1);
#pragma unroll
            for (int i = 0; i < kFMe * kFNe; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            mma_sub(1);
            __builtin_amdgcn_sched_barrier(0);
            if (grp == 0)
                wait_vmcnt<T::kDma>();
            barrier();
        }
        if (grp == 0)
            barrier();
    } else if constexpr (!T::kAhead) {
    // ---- prologue: stages 0 .. STAGES-2 in flight, stage 0 landed ----
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        issue_stage(st, 0, 1);
    wait_stage();
    __syncthreads();
    read_b(0, 0, 0);
    read_a(0, 0, 0);
    asm volatile("" ::: "memory");

    // ---- main loop (branch-free body) ----
    // Sub-step ks runs the matrix cores on (fa[ks&1], bop[ks&1]) while the
    // fragments of ks+1 are read and unpacked into the other slots (the first
    // sub-step's B operands are unpacked at its start, fragment by fragment).
    for (int step = 0; step < steps; ++step) {

#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int cur = ks & 1;
            if (ks == 0)
                unpack_b(0, 0);  // this stage's first B operands (read after the last barrier)
            if (ks < 3) {
                if ((ks + 1) % T::kSPR == 0)
                    read_b(step, (ks + 1) / T::kSPR, ((ks + 1) / T::kSPR) & 1);
                read_a(step, ks + 1, cur ^ 1);
                // a third of the loads for stage step+STAGES-1 (zeros past K)
                issue_stage(step + STAGES - 1, ks, 3);
                mfma_rows(cur, cur, 0, T::kFM);
                unpack_b(ks + 1, cur ^ 1);
                // all of the next sub-step's reads first (they have a whole
                // sub-step to land), then the matrix work with the unpack
                // of the next B operands interleaved
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReads, 0);
#pragma unroll
                for (int i = 0; i < T::kFM * T::kFN; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                mfma_rows(cur, cur, 0, kHalf);
                __builtin_amdgcn_sched_barrier(0);
                // stage step+1 has landed (only the loads issued this step may
                // still be in flight) and every wave is done with stage step
                wait_stage();
                __syncthreads();
                read_b(step + 1, 0, 0);
                read_a(step + 1, 0, 0);
                mfma_rows(cur, cur, kHalf, T::kFM);
#pragma unroll
                for (int i = 0; i < kReads; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" ::: "memory");
            }
        }
    }
    } else {
        // ---- stage-ahead loop (32 x 32 wave tiles): a wave's operands for a
        // whole stage are read right after the barrier that publishes the
        // stage, one step before they are used.  With a ring of six stages or
        // more a step covers two stages (SPS), so one barrier serves two.
        constexpr int kPk = 4 / T::kSPR;  // packed B reads per stage
        constexpr int SPS = STAGES >= 6 ? 2 : 1;
        v4i ga[2][SPS][4][T::kFM];
        uint4 gb[2][SPS][kPk][T::kFN];
        auto read_stage = [&](int step, int slot, int u) {
            const int8_t *la = lds + (step % STAGES) * T::kStage;
            const int8_t *lb = la + T::kSA;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int chunk = (2 * (ks / T::kSPR) + fg) * T::kSPR + ks % T::kSPR;
#pragma unroll
                for (int i = 0; i < T::kFM; ++i) {
                    const int row = wm * T::kWM + i * 32 + fr;
                    ga[slot][u][ks][i] = *(const v4i *)(la + row * kBK + ((chunk ^ swz<T::kGrayA>(row, 1, 7)) * 16));
                }
            }
#pragma unroll
            for (int q = 0; q < kPk; ++q) {
                const int chunk = 2 * q + fg;
#pragma unroll
                for (int j = 0; j < T::kFN; ++j) {
                    const int row = wn * T::kWN + j * 32 + fr;
                    gb[slot][u][q][j] = *(const uint4 *)(lb + row * T::kPB +
                                                         ((chunk ^ swz<false>(row, T::kSwzShiftB, T::kCPR - 1)) * 16));
                }
            }
        };
        auto compute_stage = [&](int slot, int u) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                v4i bo[T::kFN];
#pragma unroll
                for (int j = 0; j < T::kFN; ++j) {
                    if constexpr (NF4)
                        bo[j] = decode_nf4(dword_of(gb[slot][u][0][j], ks), lut[j]);
                    else
                        bo[j] = U::operand_rt(gb[slot][u][ks / T::kSPR][j], ks % T::kSPR);
                }
#pragma unroll
                for (int j = 0; j < T::kFN; ++j)
#pragma unroll
                    for (int i = 0; i < T::kFM; ++i)
                        acc[i][j] = mma32<NF4>(ga[slot][u][ks][i], bo[j], acc[i][j]);
            }
        };
        // One step (stages step .. step+SPS-1): stages step+SPS ..
        // step+2SPS-1 landed (of the stages issued so far, through
        // step+STAGES-SPS-1, the last STAGES-3SPS may still be in flight) and
        // this wave's reads of two steps ago done, then the barrier; after it,
        // the loads of stages step+STAGES-SPS .. step+STAGES-1 go into the
        // slots those reads used, the operands of the next step's stages are
        // read and this step's stages are computed from the operands read one
        // step ago.  Only the reads of two steps ago are waited for at the
        // barrier (all but the last 15 when a step reads more), so the latest
        // reads stay in flight across it.  The scheduling fences keep the
        // unpack of the operands just read (register work) from being hoisted
        // next to the reads.  Steps are unrolled by two so the operand slots
        // are compile-time register indices; in the last steps, stages past
        // the end are read (in range, never used) but not computed.
        constexpr int kReadsStage = 4 * T::kFM + kPk * T::kFN;
        constexpr int kReadsStep = SPS * kReadsStage < 15 ? SPS * kReadsStage : 15;
        auto one_step = [&](int step, int cur, bool full) {
            if constexpr (T::kEvenA && T::kEvenB)
                wait_vmcnt<(STAGES - 3 * SPS) * T::kDma>();
            else
                wait_vmcnt_rt<STAGES - 3 * SPS, T::kDma>(myDma);
            wait_lgkmcnt<kReadsStep>();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < SPS; ++u)
                issue_stage(step + STAGES - SPS + u, 0, 1);
#pragma unroll
            for (int u = 0; u < SPS; ++u)
                read_stage(step + SPS + u, cur ^ 1, u);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < SPS; ++u)
                if (full || step + u < steps)
                    compute_stage(cur, u);
            __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll
        for (int st = 0; st < STAGES - SPS; ++st)
            issue_stage(st, 0, 1);
        // the first SPS stages landed: of STAGES-SPS issued, STAGES-2SPS may be in flight
        if constexpr (T::kEvenA && T::kEvenB)
            wait_vmcnt<(STAGES - 2 * SPS) * T::kDma>();
        else
            wait_vmcnt_rt<STAGES - 2 * SPS, T::kDma>(myDma);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < SPS; ++u)
            read_stage(u, 0, u);
        // both halves unconditional inside the loop, so the accumulators keep
        // their registers across it; the last one or two steps run after it
        int step = 0;
        for (; step + 2 * SPS <= steps; step += 2 * SPS) {
            one_step(step, 0, true);
            one_step(step + SPS, 1, true);
        }
        if (step < steps)
            one_step(step, 0, false);
        if (step + SPS < steps)
            one_step(step + SPS, 1, false);
    }

    // The loads issued in the last steps (zeros past K) must land before LDS
    // is reused or the wavefront ends.
    wait_vmcnt<0>();

    if constexpr (SPLIT) {
        // Exchange of the partial sums through the caller's workspace, ordered
        // by the AMDGPU memory model at agent scope (the XCDs' L2 caches are
        // not coherent with each other): every workgroup stores its sums
        // (lane-major, coalesced 16-byte stores), and each wavefront then
        // executes an agent-scope release fence (buffer_wbl2 sc1 and
        // s_waitcnt vmcnt(0): its stores are written back from this XCD's L2
        // and complete) before the barrier after which one thread counts the
        // arrival with an agent-scope atomic add.  The last workgroup of the
        // tile to arrive executes an agent-scope acquire fence in every
        // wavefront (buffer_inv sc1: later loads miss this XCD's L2) after the
        // barrier that publishes the count, then loads the other parts' sums
        // and adds them to its own.  This is the fence - barrier - atomic
        // pattern of a grid-wide reduction, with the release half paid by every
        // workgroup and the acquire half only by the last.
        constexpr int kQ = T::kFM * T::kFN * 4;  // 16-byte pieces per lane
        const int64_t tile0 = (int64_t)t * sk.parts * kQ * kThreads + tid;
        int4 *mine = sk.part + tile0 + (int64_t)split * kQ * kThreads;
#pragma unroll
        for (int i = 0; i < T::kFM; ++i)
#pragma unroll
            for (int j = 0; j < T::kFN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    mine[((i * T::kFN + j) * 4 + q) * kThreads] =
                        make_int4((int)bits32(acc[i][j][4 * q]), (int)bits32(acc[i][j][4 * q + 1]),
                                  (int)bits32(acc[i][j][4 * q + 2]), (int)bits32(acc[i][j][4 * q + 3]));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        __shared__ int lastArrival;
        if (tid == 0) {
            const int arrived = __hip_atomic_fetch_add(sk.ctr + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
            lastArrival = arrived == sk.parts;
            if (arrived == sk.parts)  // ready for the next launch
                __hip_atomic_store(sk.ctr + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!lastArrival)
            return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        for (int p = 0; p < sk.parts; ++p) {
            if (p == split)
                continue;
            const int4 *other = sk.part + tile0 + (int64_t)p * kQ * kThreads;
#pragma unroll
            for (int i = 0; i < T::kFM; ++i)
#pragma unroll
                for (int j = 0; j < T::kFN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int4 v = other[((i * T::kFN + j) * 4 + q) * kThreads];
                        const int w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (NF4)
                                acc[i][j][4 * q + e] += __uint_as_float((uint32_t)w[e]);
                            else
                                acc[i][j][4 * q + e] += w[e];
                        }
                    }
        }
    }

    // ---- epilogue ----
    // Accumulator layout: lane l of a 32 x 32 fragment acc[i][j] holds
    // column n = wn*kWN + 32 j + (l & 31) and, in registers 4g..4g+3, the
    // four consecutive rows m = wm*kWM + 32 i + 8 g + 4 (l >> 5) + (0..3); of
    // a 16 x 16 fragment (the ping-pong loop), column wn*kWN + 16 j + (l & 15)
    // and rows wm*kWM + 16 i + 4 (l >> 4) + (0..3): in both, groups of four
    // consecutive rows of one column.
    // Both output types are staged through LDS, 64 rows (or fewer) of each
    // wave's tile at a time, and written as whole 16-byte chunks of rows.
    {
        constexpr int kPerChunk = 16 / T::kES;           // outputs per 16-byte chunk
        const bool vecN = (N % kPerChunk) == 0;
        __syncthreads();  // every wave is done with the stage buffers
        int8_t *stg = lds + wave * T::kEpiRows * T::kEpiPitch;
        constexpr int kChunksPerRow = T::kWN / kPerChunk;  // 16-byte chunks per staged row
        constexpr int kRowsPerIt = 64 / kChunksPerRow;
        constexpr int kFragsPerPass = T::kEpiRows / kCF;
        constexpr int kG = kM16 ? 1 : 4;  // groups of four rows per lane and fragment
        static_assert(kG * 4 == (int)(sizeof(AccE) / 4), "a lane's accumulator holds kG groups of four rows");
        // the first of a group's four rows, fragment-local
        auto grow = [&](int g) { return kM16 ? 4 * (lane >> 4) : 8 * g + 4 * fg; };
        const int fcol = kM16 ? (lane & 15) : fr;  // the lane's column, fragment-local
        static_assert(kChunksPerRow <= 16 && 16 % kChunksPerRow == 0 && T::kEpiRows % kRowsPerIt == 0,
                      "epilogue copy-out shape");
        // Copy-out: each 16 consecutive lanes read 16 / kChunksPerRow whole
        // rows, spaced by kRowGap so that, with the 32-byte row padding, their
        // 16-byte chunks fall in 16 distinct 16-byte bank groups.  (The
        // hardware serves a 16-byte read in other 16-lane groups, see swz(),
        // under which some groups still meet twice; the copy-out is a few
        // reads per tile, so that costs nothing measurable.)
        constexpr int kRowsPer16 = 16 / kChunksPerRow;
        constexpr int kRowGap = kRowsPer16 == 4 ? 2 : kRowsPer16 == 2 ? 4 : 1;
        const int q16 = lane >> 4;
        const int outRow = (q16 / kRowGap) * (kRowGap * kRowsPer16) + q16 % kRowGap +
                           kRowGap * ((lane & 15) / kChunksPerRow);
        const int outChunk = lane % kChunksPerRow;
        const bool oddLane = (lane & 1) != 0;
        // the passes, with the activation and the presence of token scales
        // fixed at compile time (a per-element choice would keep the compiler
        // from interleaving the elements' dependent chains)
        auto passes = [&](auto actTag, auto xsTag) {
            constexpr int kAct = decltype(actTag)::value;
            constexpr bool kXs = FUSE && decltype(xsTag)::value;
#pragma unroll
            for (int i0 = 0; i0 < kFMe; i0 += kFragsPerPass) {
                // with token scales, those of the lane's rows of this pass
                // (four consecutive rows per 8-byte load: m is a multiple of 4)
                float xs[kXs ? kFragsPerPass : 1][kG][4];
                if constexpr (kXs) {
#pragma unroll
                    for (int ii = 0; ii < kFragsPerPass; ++ii)
#pragma unroll
                        for (int g = 0; g < kG; ++g) {
                            const int m = m0 + wm * T::kWM + (i0 + ii) * kCF + grow(g);
                            uint32_t h[4];
                            if (m + 4 <= M) {
                                const uint2 p = *(const uint2 *)(xscale + m);
                                h[0] = p.x & 0xFFFF; h[1] = p.x >> 16; h[2] = p.y & 0xFFFF; h[3] = p.y >> 16;
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    h[e] = m + e < M ? xscale[m + e] : 0u;
                            }
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                xs[ii][g][e] = __half2float(__ushort_as_half((unsigned short)h[e]));
                        }
                }
#pragma unroll
                for (int j = 0; j < kFNe; ++j) {
                    const int nl = j * kCF + fcol;  // the lane's column, wave-local
#pragma unroll
                    for (int ii = 0; ii < kFragsPerPass; ++ii) {
                        const int i = i0 + ii;
#pragma unroll
                        for (int g = 0; g < kG; ++g) {
                            const int r = ii * kCF + grow(g);  // first of the 4 rows, pass-local
                            if constexpr (F16OUT) {
                                // weight scale, times the row's activation scale with
                                // FUSE (a product of two fp16 values, exact in fp32),
                                // then the activation
                                float v[4];
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    if constexpr (NF4)
                                        v[e] = acc[i][j][4 * g + e];  // the scale is in the weights
                                    else
                                        v[e] = (float)acc[i][j][4 * g + e] * (kXs ? sc[j] * xs[ii][g][e] : sc[j]);
                                    v[e] = act_fixed<kAct>(v[e]);
                                }
                                // rows (r, r+1) and (r+2, r+3) of column nl as fp16 pairs;
                                // the even lane of each pair of columns keeps rows r, r+1
                                // and takes those of its odd neighbour, which keeps
                                // rows r+2, r+3, so each LDS write is two adjacent
                                // columns of one row (DPP quad_perm [1,0,3,2]: lane ^ 1)
                                const h2v p01 = {(_Float16)v[0], (_Float16)v[1]};
                                const h2v p23 = {(_Float16)v[2], (_Float16)v[3]};
                                const uint32_t x01 = __builtin_bit_cast(uint32_t, p01);
                                const uint32_t x23 = __builtin_bit_cast(uint32_t, p23);
                                const uint32_t keep = oddLane ? x23 : x01;
                                const uint32_t got =
                                    (uint32_t)__builtin_amdgcn_mov_dpp((int)(oddLane ? x01 : x23), 0xB1, 0xF, 0xF, false);
                                const uint32_t lo = oddLane ? got : keep;   // the even column
                                const uint32_t hi = oddLane ? keep : got;   // the odd column
                                const int rr = r + (oddLane ? 2 : 0);
                                int8_t *p = stg + rr * T::kEpiPitch + (nl & ~1) * 2;
                                *(uint32_t *)p = (lo & 0xFFFFu) | (hi << 16);
                                *(uint32_t *)(p + T::kEpiPitch) = (lo >> 16) | (hi & 0xFFFF0000u);
                            } else {
                                // exact: the sums are multiples of 2^kShift
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    *(int *)(stg + (r + e) * T::kEpiPitch + nl * 4) = acc[i][j][4 * g + e] >> U::kShift;
                            }
                        }
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int it = 0; it < T::kEpiRows / kRowsPerIt; ++it) {
                    const int r = it * kRowsPerIt + outRow;
                    const uint4 v = *(const uint4 *)(stg + r * T::kEpiPitch + outChunk * 16);
                    const int m = m0 + wm * T::kWM + i0 * kCF + r;
                    const int n = n0 + wn * T::kWN + outChunk * kPerChunk;
                    if (m < M && n < N) {
                        void *dst = (int8_t *)C + ((int64_t)m * N + n) * T::kES;
                        if (vecN && n + kPerChunk <= N) {
                            // streaming store: the output is not read again by
                            // this kernel, and lines marked so leave L2 early
                            // instead of being written back at the kernel's end
                            // (M = N = K = 4096: 57.7 against 59.0 us)
                            __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), (v4i *)dst);
                        } else {
                            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                            if constexpr (F16OUT) {
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    if (n + e < N)
                                        ((uint16_t *)dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (n + e < N)
                                        ((uint32_t *)dst)[e] = w[e];
                            }
                        }
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);
                __builtin_amdgcn_wave_barrier();
            }
        };
        auto with_act = [&](auto xsTag) {
            if (act == 2)
                passes(std::integral_constant<int, 2>{}, xsTag);
            else if (act == 1)
                passes(std::integral_constant<int, 1>{}, xsTag);
            else
                passes(std::integral_constant<int, 0>{}, xsTag);
        };
        if constexpr (FUSE) {
            if (xscale)
                with_act(std::true_type{});
            else
                with_act(std::false_type{});
        } else {
            passes(std::integral_constant<int, 0>{}, std::false_type{});
        }
    }
}

template <int BITS, int BM, int BN, int STAGES, int WAVES, bool SPLIT = false, bool NF4 = false, int WGM = 2>
hipError_t launch_t(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale,
                    int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s,
                    const SplitK &sk = {})
{
    const int64_t tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
    const int64_t wgs = tilesM * tilesN * (SPLIT ? sk.parts : 1);
    if (!grid_fits(wgs, 64 * WAVES))
        return kGridTooLarge;
    const dim3 grid((unsigned)wgs, (unsigned)batch);
    const bool tail = (K % kBK) != 0;
#define BQ_TILED_LAUNCH(F16, TAIL, FUSED)                                                                   \
    gemm_tiled_kernel<BITS, BM, BN, STAGES, F16, TAIL, WAVES, FUSED, SPLIT, NF4, WGM><<<grid, 64 * WAVES, 0, s>>>( \
        A, B, scale, xscale, act, C, M, N, K, (int)tilesM, (int)tilesN, bs, sk)
    if constexpr (NF4) {
        // the row width of A is a whole number of 128-byte stages (K % 64 == 0)
        BQ_TILED_LAUNCH(true, false, false);
    } else if (scale && (xscale || act != 0)) {
        if (tail)
            BQ_TILED_LAUNCH(true, true, true);
        else
            BQ_TILED_LAUNCH(true, false, true);
    } else if (scale) {
        if (tail)
            BQ_TILED_LAUNCH(true, true, false);
        else
            BQ_TILED_LAUNCH(true, false, false);
    } else {
        if (tail)
            BQ_TILED_LAUNCH(false, true, false);
        else
            BQ_TILED_LAUNCH(false, false, false);
    }
#undef BQ_TILED_LAUNCH
    return hipGetLastError();
}

// Tile configuration by the number of output tiles; the 256 CUs want a few
// hundred workgroups.  Measured on MI355X at N = K = 4096 (W4A8):
//  * 256 x 256, eight wavefronts (2 x 4 of 128 x 64), once there are 256
//    such tiles (M >= 4096);
//  * 128 x 128 from 192 tiles (M >= 768), eight wavefronts (64 x 32 each)
//    for int4, four for int8 (64 x 64) and int2 (128 x 32): W4A8 22 us at
//    M = 768 and 25 us at M = 1024 (24 / 27.6 with four wavefronts), 43 us at
//    M = 2048 where the 256 x 256 tiles take 49; W2A8 24.4 us at M = 1024
//    (27.8 with eight 64 x 32 wave tiles);
//  * 64 x 64, four wavefronts (32 x 32 each), a 4-stage ring, from 512 tiles
//    (several workgroups per CU; 17 us at M = 512, against 22 us with
//    128 x 128 tiles);
//  * 64 x 64 with an 8-stage ring below that (11.1 us at M = 128, 12.2 us at
//    M = 256, 15 us for W8A8 at M = 64, N = 12288; 21 us with 128 x 128);
//    with at most 128 such tiles (half the CUs or fewer), K is split over
//    2-8 workgroups per tile (SplitK) so that up to 256 workgroups run
//    (M = 64: 11.0 -> 10.0 us; M = 128: 11.1 -> 10.4 us, W2A8 14.4 -> 11.9 us,
//    W8A8 12.5 -> 11.0 us).

// K split over workgroups: only with a workspace from the caller (the
// library allocates nothing).  The workspace holds the per-tile counters
// (kCtrBytes, zero before the first use; every launch leaves them zero) and
// then the partial sums of at most kSplitMaxWgs workgroups.
constexpr int kSplitMaxTiles = 128;   // split only with this many tiles or fewer
constexpr int kSplitMaxWgs = 256;     // tiles x parts
constexpr int kSplitMaxParts = 8;
constexpr int kSplitMinSteps = 4;     // 128-k stages per workgroup, at least
constexpr int64_t kCtrBytes = 4096;
constexpr int64_t kPartBytesPerWg = 256 * 16 * 4;  // 256 threads x 16 int32 each

// Parts of the K split for a shape (1: no split).
int split_parts(int M, int N, int K, int batch)
{
    const int64_t t64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
    const int64_t t128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    if (batch != 1 || t64 > kSplitMaxTiles || t128 >= 192 || t64 >= 512)
        return 1;
    const int stepsAll = (K + kBK - 1) / kBK;
    const int parts = min(kSplitMaxParts, min(kSplitMaxWgs / (int)t64, stepsAll / kSplitMinSteps));
    if (parts < 2)
        return 1;
    // equal stage counts; the rounding never leaves a workgroup empty
    const int per = (stepsAll + parts - 1) / parts;
    return (stepsAll + per - 1) / per;
}

template <int BITS, bool NF4 = false>
hipError_t launch_bits(const int8_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *xscale,
                       int act, void *C, int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s,
                       void *ws, int64_t wsBytes)
{
    // Three LDS stages fit in 160 KB except for 256x256 int8 (64 KB per stage).
    constexpr int kStages256 = BITS == 8 ? 2 : 3;
    const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    const int64_t t64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
    if (t256 >= 256)
        // NF4: a 1 x 8 wavefront grid (256 x 32 each), so each B column's
        // codes are decoded by one wavefront instead of two
        return launch_t<BITS, 256, 256, kStages256, 8, false, NF4, NF4 ? 1 : 2>(A, B, scale, xscale, act, C, M, N, K,
                                                                               batch, bs, s);
    // 128 x 128: int4 eight wavefronts (2 x 4 of 64 x 32); int8 four (2 x 2
    // of 64 x 64); int2 and NF4 four in a 1 x 4 grid (128 x 32 each), so each
    // B column is unpacked or decoded by one wavefront
    constexpr int kWaves128 = BITS == 4 ? 8 : 4;
    constexpr int kWgm128 = BITS == 2 ? 1 : 2;
    // 64 x 64: four wavefronts (2 x 2 of 32 x 32); NF4 two (1 x 2 of 64 x 32)
    constexpr int kWaves64 = NF4 ? 2 : 4;
    if (t128 >= 192)
        return launch_t<BITS, 128, 128, 3, kWaves128, false, NF4, kWgm128>(A, B, scale, xscale, act, C, M, N, K, batch,
                                                                          bs, s);
    if (t64 >= 512)
        return launch_t<BITS, 64, 64, 4, kWaves64, false, NF4, NF4 ? 1 : 2>(A, B, scale, xscale, act, C, M, N, K,
                                                                           batch, bs, s);
    const int parts = ws ? split_parts(M, N, K, batch) : 1;
    if (parts >= 2 && wsBytes >= kCtrBytes + t64 * parts * kPartBytesPerWg) {
        SplitK sk;
        sk.parts = parts;
        sk.stepsPer = ((K + kBK - 1) / kBK + parts - 1) / parts;
        sk.ctr = (int *)ws;
        sk.part = (int4 *)((char *)ws + kCtrBytes);
        return launch_t<BITS, 64, 64, 8, kWaves64, true, NF4, NF4 ? 1 : 2>(A, B, scale, xscale, act, C, M, N, K, 1, bs,
                                                                          s, sk);
    }
    return launch_t<BITS, 64, 64, 8, kWaves64, false, NF4, NF4 ? 1 : 2>(A, B, scale, xscale, act, C, M, N, K, batch,
                                                                         bs, s);
}

}  // namespace

int64_t gemm_splitk_workspace_bytes(int M, int N, int K, int bits)
{
    (void)bits;
    const int parts = split_parts(M, N, K, 1);
    if (parts < 2)
        return 0;
    const int64_t t64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
    return kCtrBytes + t64 * parts * kPartBytesPerWg;
}

hipError_t launch_gemm_nf4(const uint16_t *A, const uint8_t *B, const uint16_t *scale, const uint16_t *zero,
                           uint16_t *C, int M, int N, int K, hipStream_t s)
{
    if (M == 0 || N == 0)
        return hipSuccess;
    // in the kernel's byte terms an A row is 2K bytes wide (see the kernel)
    return launch_bits<2, true>((const int8_t *)A, B, scale, zero, 0, C, M, N, 2 * K, 1, {}, s, nullptr, 0);
}

hipError_t launch_gemm_tiled(const int8_t *A, const uint8_t *B, int bits,
                             const uint16_t *scale, const uint16_t *xscale, int act, void *C,
                             int M, int N, int K, int batch, const BatchStrides &bs, hipStream_t s,
                             void *ws, int64_t wsBytes)
{
    if (M == 0 || N == 0)
        return hipSuccess;
    switch (bits) {
    case 8: return launch_bits<8>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s, ws, wsBytes);
    case 4: return launch_bits<4>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s, ws, wsBytes);
    default: return launch_bits<2>(A, B, scale, xscale, act, C, M, N, K, batch, bs, s, ws, wsBytes);
    }
}

}  // namespace bq
