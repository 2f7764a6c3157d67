/*
 * bq.h - C ABI of the MI355X (gfx950) quantized GEMM library libbq.so.
 *
 * The library implements one hot path of low-bit LLM inference:
 *
 *   1. per-row symmetric int8 quantization of an fp16 matrix
 *      (scale = absmax/127 as fp16, codes = nearest integer of x/scale);
 *   2. packing of int8-held int4 / int2 weight values into bytes along K;
 *   3. the mixed-precision GEMM
 *        acc[m,n] = sum_k A[m,k] * B[n,k]            (int32)
 *        C[m,n]   = fp16(acc[m,n] * scale[n])        (optional epilogue)
 *      with A int8 [M,K] and B int8, int4 or int2 [N,K].
 *
 * Sources (page title, section):
 *  - "BMINF的後訓練量化實現" (BMINF post-training quantization), 實現代碼分析2:
 *    the quantize(x, out, scale, axis) contract and its two kernels
 *    (per-row absmax/127 reduction, nearest-integer copy to int8), the
 *    int8 weight [out, in] with fp16 scale [out, 1] parameter layout, and
 *    the caller-allocated outputs of PartialAttention.quantize;
 *  - "BitBLAS自定义操作开发指南：使用DSL扩展新的混合精度算子" (BitBLAS custom
 *    operator guide), sections 1-2 and cases 1-2: int8 x int4 / int2 matmul
 *    with int32 accumulation over K of B stored [N, K], dequantization by a
 *    per-N fp16 scale with arguments ordered (A, B, scale, C), sub-byte
 *    weights stored compressed as uint8 [N, K/2], and a dynamic range of M.
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is a HIP DEVICE pointer owned by the caller; the
 *    library never frees or retains caller pointers.  Outputs must not
 *    alias inputs.
 *  - Every buffer is dense, row-major (C-contiguous) and 16-byte aligned.
 *  - fp16 data is passed as void* holding IEEE binary16 bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous: they validate, enqueue kernels on `stream` and return;
 *    the caller synchronizes.  A call on a stream is ordered with the
 *    caller's other work on that stream.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued; a nonzero status means nothing was enqueued, except
 *    BQ_ERR_HIP, which reports a failed launch.  Nothing aborts or throws
 *    across the ABI.  A dimension of 0 (other than K) is a valid no-op.
 *  - The device must be gfx950 (BQ_ERR_DEVICE otherwise); the check is made
 *    once per device.
 *  - Library memory: the library allocates no device memory, frees none and
 *    keeps no pointer past a call (BMINF page, 實現代碼分析2: the caller
 *    allocates every output, the kernels only fill it).  The one call that
 *    uses scratch memory, bq_gemm_splitk, takes it from the caller.
 *  - Grid limits: a launch counts work-items per grid dimension and the
 *    count must stay below 2^32; a shape whose launch would exceed it returns
 *    BQ_ERR_SHAPE with nothing enqueued (e.g. bq_quantize_rows with 2^24 or
 *    more rows, whose kernel runs 256 work-items per row).
 *  - Thread safety: calls are reentrant; the only shared state is a cached
 *    per-device property record, written once.
 */
#ifndef BQ_H
#define BQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bq_status {
    BQ_OK = 0,
    BQ_ERR_NULL = 1,   /* a required pointer is NULL                          */
    BQ_ERR_SHAPE = 2,  /* negative dimension, or a divisibility / size limit  */
    BQ_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned                    */
    BQ_ERR_HIP = 4,    /* a HIP runtime call or kernel launch failed          */
    BQ_ERR_DEVICE = 5, /* the current device is not gfx950                    */
    BQ_ERR_ARG = 6     /* an enumerated argument (bits, path) is invalid      */
};

/* Largest K accepted by the GEMMs.  With int8 operands the int32 sum is
 * bounded by K * 128 * 128, which stays below 2^31 for K <= 131071; the
 * limit leaves a factor of two of headroom. */
#define BQ_MAX_K 65536

/* Largest M and N accepted by the GEMMs, and the largest output M * N: the
 * kernels index rows and tiles in 32-bit integers, which these bounds keep
 * exact.  An output at the limit holds 2^42 elements (8 TiB in fp16), more
 * than one device's memory.  Within them, a shape whose grid would exceed
 * the dispatch limit (see the conventions) is rejected with BQ_ERR_SHAPE. */
#define BQ_MAX_DIM (1LL << 30)
#define BQ_MAX_OUT (1LL << 42)

/* GEMM path selection for bq_gemm (the named GEMM calls use BQ_PATH_AUTO). */
enum bq_path {
    BQ_PATH_AUTO = 0,   /* choose by M (see bq_gemm_select_path)              */
    BQ_PATH_STREAM = 1, /* streaming matrix-core kernel, M <= 256 (auto: 3 <= M <= 128, int2 <= 256) */
    BQ_PATH_TILED = 2,  /* LDS-tiled matrix-core kernel, any M                */
    BQ_PATH_GEMV = 3    /* decode GEMV on dot-product ALUs, M <= 4 (auto: M <= 2) */
};

/* Library version as an integer (major*10000 + minor*100 + patch). */
int bq_version(void);

/* Static, NUL-terminated description of a status code. */
const char *bq_status_string(int status);

/*
 * bq_quantize_rows - per-row symmetric int8 quantization.
 * BMINF page, 實現代碼分析2, quantize() docstring (kernels
 * bms_quantize_scale and bms_quantize_copy_half), reading: the code is the
 * nearest integer to the EXACT quotient x/scale with ties to even, clamped
 * to [-127, 127]; a row whose scale rounds to 0 gets codes 0.
 *
 *   x_f16     [rows, cols] fp16 input (finite values; NaN/Inf give
 *             unspecified codes for that row)
 *   q         [rows, cols] int8 output codes
 *   scale_f16 [rows]       fp16 output, fp16(absmax_row / 127) rounded to
 *                          nearest even
 * rows, cols >= 0.  cols == 0 writes scale 0 for every row.
 * Any cols is accepted; 16-byte alignment is required of x and q.
 */
int bq_quantize_rows(const void *x_f16, int64_t rows, int64_t cols,
                     int8_t *q, void *scale_f16, void *stream);

/*
 * bq_quantize_rows_bits - bq_quantize_rows with the code range of a weight
 * format: qmax = 2^(bits-1) - 1 (127, 7 or 1 for bits 8, 4, 2), scale_f16 =
 * fp16(absmax_row / qmax), codes clamped to [-qmax, qmax] (the BMINF page's
 * per-row rule, section 實現代碼分析2, with the int4 / ternary code range; the
 * codes feed bq_pack_int4 / bq_pack_int2 directly).
 *   bits  8, 4 or 2 (BQ_ERR_ARG otherwise); other arguments, layouts and
 *         errors as for bq_quantize_rows.
 */
int bq_quantize_rows_bits(const void *x_f16, int64_t rows, int64_t cols, int bits, int8_t *q,
                          void *scale_f16, void *stream);

/*
 * bq_quantize_pack - bq_quantize_rows_bits (bits 4 or 2) with the codes
 * written straight in the packed storage of bq_pack_int4 / bq_pack_int2
 * (BMINF page, 實現代碼分析2, per-row rule with the int4 / ternary code range;
 * BitBLAS guide, cases 1-2, packed weight storage): one pass over the fp16
 * weight, no int8 codes in memory.  The packed bytes and scales equal those
 * of bq_quantize_rows_bits followed by bq_pack_int4 / bq_pack_int2.
 *
 *   x_f16     [rows, cols] fp16 input
 *   bits      4 or 2 (BQ_ERR_ARG otherwise)
 *   packed    [rows, cols*bits/8] uint8 output
 *   scale_f16 [rows] fp16 output, fp16(absmax_row / qmax), qmax = 7 or 1
 * cols must be a multiple of 8/bits (BQ_ERR_SHAPE otherwise); rows, cols >= 0;
 * x, packed and scale 16-byte aligned.  Other errors as bq_quantize_rows.
 */
int bq_quantize_pack(const void *x_f16, int64_t rows, int64_t cols, int bits, uint8_t *packed,
                     void *scale_f16, void *stream);

/*
 * bq_pack_int4 - pack int4 values held one per int8 into bytes along K.
 * BitBLAS guide, case 2 (uint8 [N, K/2] compressed storage); bit order:
 * byte [n, k/2] = (v[n,k] & 0xF) | (v[n,k+1] & 0xF) << 4 for even k.
 *
 *   v   [n, k]   int8 values, expected in [-8, 7]; for values outside that
 *                range the low four bits are stored
 *   out [n, k/2] uint8
 * k must be even (BQ_ERR_SHAPE otherwise).
 */
int bq_pack_int4(const int8_t *v, int64_t n, int64_t k, uint8_t *out, void *stream);

/*
 * bq_pack_int2 - pack 2-bit (BitNet-b1.58 ternary) values along K.
 * BitBLAS guide, case 1 (int2 weights); bit order: byte [n, k/4] holds the
 * code v[n, k+j] + 2 in bits 2j..2j+1, j = 0..3 (lowest bits = lowest k).
 *
 *   v   [n, k]   int8 values, expected in [-2, 1] (ternary data: -1, 0, 1);
 *                outside that range the low two bits of v+2 are stored
 *   out [n, k/4] uint8
 * k must be a multiple of 4.
 */
int bq_pack_int2(const int8_t *v, int64_t n, int64_t k, uint8_t *out, void *stream);

/*
 * bq_gemm_w{8,4,2}a8_dequant - C = fp16((A . B^T as int32) * scale[n]).
 * BitBLAS guide, section 2 (create_dequantize_matmul), arguments in its
 * order (A, B, scale, C).  The epilogue multiplies in fp32 and rounds to
 * fp16 once (nearest even): the result is within one fp16 ulp of the
 * correctly rounded product, and |acc*scale| >= 65520 gives +-inf.
 *
 *   A         [M, K]            int8, row-major
 *   B         w8: int8 [N, K];  w4: uint8 [N, K/2] (bq_pack_int4 layout);
 *             w2: uint8 [N, K/4] (bq_pack_int2 layout)
 *   scale_f16 [N]               fp16
 *   C_f16     [M, N]            fp16 output, row-major
 * 0 <= M, N <= BQ_MAX_DIM, M * N <= BQ_MAX_OUT; 0 <= K <= BQ_MAX_K and
 * K % 64 == 0 (an implementation limit; pad K with zero columns of A
 * otherwise).  K == 0 writes zeros.
 */
int bq_gemm_w8a8_dequant(const int8_t *A, const int8_t *B, const void *scale_f16,
                         void *C_f16, int64_t M, int64_t N, int64_t K, void *stream);
int bq_gemm_w4a8_dequant(const int8_t *A, const uint8_t *B, const void *scale_f16,
                         void *C_f16, int64_t M, int64_t N, int64_t K, void *stream);
int bq_gemm_w2a8_dequant(const int8_t *A, const uint8_t *B, const void *scale_f16,
                         void *C_f16, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * bq_gemm_w{8,4,2}a8_i32 - C = A . B^T with the int32 accumulator as output.
 * BitBLAS guide, section 1 and case 1 (create_mixed_precision_matmul,
 * create_bitnet_int2_matmul).  Same operand layouts and limits as above;
 * C_i32 [M, N] int32 row-major.  Exact (integer) for every valid input.
 */
int bq_gemm_w8a8_i32(const int8_t *A, const int8_t *B, int32_t *C_i32,
                     int64_t M, int64_t N, int64_t K, void *stream);
int bq_gemm_w4a8_i32(const int8_t *A, const uint8_t *B, int32_t *C_i32,
                     int64_t M, int64_t N, int64_t K, void *stream);
int bq_gemm_w2a8_i32(const int8_t *A, const uint8_t *B, int32_t *C_i32,
                     int64_t M, int64_t N, int64_t K, void *stream);

/*
 * bq_gemm - the general form of the six GEMM calls above, with an explicit
 * kernel path (BitBLAS guide, dynamic-shape section: kernels are chosen
 * over a dynamic range of M).
 *
 *   bits       8, 4 or 2 (layout of B as above); BQ_ERR_ARG otherwise
 *   scale_f16  [N] fp16, or NULL for the int32 output
 *   C          fp16 [M, N] when scale_f16 != NULL, else int32 [M, N]
 *   path       enum bq_path; BQ_PATH_STREAM requires M <= 256, BQ_PATH_GEMV
 *              requires M <= 4 (BQ_ERR_SHAPE otherwise)
 */
int bq_gemm(const int8_t *A, const void *B, int bits, const void *scale_f16,
            void *C, int64_t M, int64_t N, int64_t K, int path, void *stream);

/*
 * bq_gemm_splitk_workspace_bytes - device workspace bq_gemm_splitk uses to
 * split K for this shape: 0 when it would not split (the output has more
 * than 128 tiles of 64 x 64, or K is shorter than 1024), else 4096 bytes of
 * per-tile counters plus 16 KiB of partial sums for each of the (at most
 * 256) workgroups, at most 4 MiB + 4 KiB in all.  Negative: -BQ_ERR_ARG or
 * -BQ_ERR_SHAPE for arguments bq_gemm would reject.  Host-only; no device
 * call.
 */
int64_t bq_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits);

/*
 * bq_gemm_splitk - bq_gemm on the tiled kernel (BQ_PATH_TILED) with K split
 * over several workgroups per output tile when the output has few tiles
 * (Pallas matmul page, blocked matmul: the K blocks of one output block are
 * independent partial sums; here up to 8 workgroups each sum a share of K,
 * and the last of a tile to finish adds the others' int32 sums, which are
 * exact, and runs the epilogue).  For shapes with few output tiles and long
 * K, where one workgroup per tile would leave most CUs idle.
 *
 *   workspace        caller-owned device memory of workspace_bytes bytes,
 *                    16-byte aligned; its first 4096 bytes must be zero
 *                    before the first call (e.g. hipMemsetAsync), and every
 *                    call leaves them zero again.  NULL with 0 bytes: K is
 *                    not split.  Fewer bytes than
 *                    bq_gemm_splitk_workspace_bytes(M, N, K, bits): K is not
 *                    split (same results).
 * Calls that share a workspace must not run concurrently (calls on one
 * stream are ordered).  Other arguments, layouts and errors as for bq_gemm;
 * a negative workspace_bytes gives BQ_ERR_SHAPE, a NULL workspace with a
 * positive size BQ_ERR_NULL.
 */
int bq_gemm_splitk(const int8_t *A, const void *B, int bits, const void *scale_f16, void *C, int64_t M,
                   int64_t N, int64_t K, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * bq_gemm_splitk_static - bq_gemm_splitk with the library's own scratch
 * instead of a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It allocates nothing: the scratch is a static device
 * array of BQ_SPLITK_STATIC_BYTES (4 MiB + 4 KiB) that every GPU the library
 * runs on holds until the process ends; its per-tile counters are cleared
 * by a small kernel on `stream` before the GEMM.  A shape whose split would
 * need more scratch than that returns BQ_ERR_SHAPE (no shape accepted by
 * bq_gemm_splitk_workspace_bytes needs more).  Every call on one GPU shares
 * that GPU's scratch: calls that may overlap (on different streams, or from
 * different threads) race and give wrong results; order them on one stream.
 * Results equal those of bq_gemm_splitk.  Other arguments, layouts and
 * errors as for bq_gemm.
 */
#define BQ_SPLITK_STATIC_BYTES (4096LL + 256LL * 16384LL)
int bq_gemm_splitk_static(const int8_t *A, const void *B, int bits, const void *scale_f16, void *C, int64_t M,
                          int64_t N, int64_t K, void *stream);

/*
 * bq_gemm_dual_scale - the GEMM of a linear layer whose activations were
 * quantized per token: A [M, K] holds the int8 codes of the M token rows
 * (bq_quantize_rows over the rows of the fp16 activations) and x_scale_f16
 * [M] their scales; then
 *   C[m,n] = fp16(acc[m,n] * w_scale[n] * x_scale[m])
 * (BMINF page, section 實現代碼分析2, PartialAttention forward: the input is
 * quantized per token, multiplied by the int8 weight, and the int32 result
 * is scaled by the weight scale of its output channel and the scale of its
 * token, out0 = in0 * in1 * in2; reading: the product is rounded once to
 * fp16, the kernels multiplying the two scales exactly in fp32 and rounding
 * the product with the accumulator before the final conversion, within one
 * fp16 ulp of the correctly rounded value).
 *
 *   bits, B, path   as for bq_gemm
 *   w_scale_f16     [N] fp16 weight scales (required)
 *   x_scale_f16     [M] fp16 token scales (required, 16-byte aligned)
 *   C_f16           fp16 [M, N]
 * Errors as for bq_gemm; a NULL scale gives BQ_ERR_NULL.
 */
int bq_gemm_dual_scale(const int8_t *A, const void *B, int bits, const void *w_scale_f16,
                       const void *x_scale_f16, void *C_f16, int64_t M, int64_t N, int64_t K,
                       int path, void *stream);

/*
 * bq_gemm_batched - `batch` GEMMs of one shape in one launch, batch z on
 *   A + z*strideA, B + z*strideB, scale + z*strideScale, C + z*strideC
 * (BMINF page, section 實現代碼分析2: igemm of the fused QKV weight
 * (3, N, K) with the activation (1, M, K), broadcast over the 3 weights,
 * into (3, M, N); then the two-scale elementwise step with the token scale
 * shared by the 3 results).
 *
 *   strides    in elements of each array: int8 elements of A, bytes of
 *              (packed) B, fp16 elements of scale, output elements of C.
 *              0 broadcasts an input to every batch; strideC >= M*N when
 *              batch > 1 (outputs must not overlap).  strideA and strideB
 *              multiples of 16, strideScale and an fp16 strideC multiples
 *              of 8, an int32 strideC a multiple of 4 (BQ_ERR_ALIGN).
 *   x_scale_f16  NULL, or [M] fp16 token scales shared by every batch
 *              (requires scale_f16; then C = fp16(acc * scale * x_scale))
 *   batch      0 .. 65535
 * Other arguments and errors as for bq_gemm.
 */
int bq_gemm_batched(const int8_t *A, int64_t strideA, const void *B, int64_t strideB, int bits,
                    const void *scale_f16, int64_t strideScale, const void *x_scale_f16,
                    void *C, int64_t strideC, int64_t batch, int64_t M, int64_t N, int64_t K,
                    int path, void *stream);

/* Activation of the fused epilogue (bq_gemm_act). */
enum bq_act {
    BQ_ACT_NONE = 0, /* identity                                               */
    BQ_ACT_RELU = 1, /* max(v, 0)                                              */
    BQ_ACT_GELU = 2  /* v * Phi(v), Phi the standard normal CDF                */
};

/*
 * bq_gemm_act - the GEMM with an activation fused into the fp16 epilogue:
 *   C[m,n] = fp16(act(acc[m,n] * w_scale[n] * x_scale[m]))
 * with x_scale NULL meaning 1 (JAX Pallas matmul page, fused-activation
 * section: the activation is applied once to the wide result of the last K
 * step, before the single downcast; BladeDISC page, CUTLASS GEMM codegen:
 * GEMM + GELU fused).  Reading: the activation acts on the dequantized value;
 * the kernels evaluate it in fp32 (GELU as v * erfc(-v / sqrt(2)) / 2) and
 * round once to fp16; outputs within one fp16 ulp of the correctly rounded
 * value.
 *
 *   act          enum bq_act (BQ_ERR_ARG otherwise)
 *   w_scale_f16  [N] fp16 (required)
 *   x_scale_f16  [M] fp16 token scales, or NULL (16-byte aligned)
 * Other arguments and errors as for bq_gemm.
 */
int bq_gemm_act(const int8_t *A, const void *B, int bits, const void *w_scale_f16,
                const void *x_scale_f16, int act, void *C_f16, int64_t M, int64_t N, int64_t K,
                int path, void *stream);

/*
 * bq_gemm_nf4_a16 - W4A16 GEMM with NF4 weight codes, fp16 activations and
 * fp32 accumulation (BitBLAS guide, case 2: A fp16 [M, K], B_nf4 uint8
 * [N, K/2], scale and zero_point fp16 [N], C = sum_k fp32(A) * fp32(W)).
 * The page leaves out the NF4 table and the dequantization; readings:
 *   table[16]  the 4-bit NormalFloat codebook (QLoRA: normal quantiles,
 *              eight positive, seven negative, and zero, scaled to [-1, 1]),
 *              held in fp16; code c selects the c-th smallest value
 *   W[n,k]     fp16(fp32(fp32(table[c] - zero[n]) * scale[n])), one fp16
 *              rounding (nearest even); zero NULL means 0
 *   C[m,n]     fp16 of sum_k A[m,k] * W[n,k] accumulated in fp32 by the
 *              matrix cores; within one fp16 ulp of the exact sum's value
 *              plus the fp32 accumulation bound K 2^-24 sum_k |A W|
 *
 *   A_f16      [M, K] fp16 row-major
 *   B          [N, K/2] uint8: code of k even in the low nibble, k odd in
 *              the high nibble (codes 0..15)
 *   scale_f16  [N] fp16 (required); zero_f16 [N] fp16 or NULL
 *   C_f16      [M, N] fp16
 * 0 <= M, N <= BQ_MAX_DIM, M * N <= BQ_MAX_OUT; 0 <= K <= BQ_MAX_K,
 * K % 64 == 0 (BQ_ERR_SHAPE); pointers
 * 16-byte aligned (BQ_ERR_ALIGN); NULL where required (BQ_ERR_NULL).  M <= 4
 * runs a decode GEMV (dot products on the vector ALUs, a stream over B);
 * larger M the tiled matrix-core kernel.
 */
int bq_gemm_nf4_a16(const void *A_f16, const uint8_t *B, const void *scale_f16, const void *zero_f16,
                    void *C_f16, int64_t M, int64_t N, int64_t K, void *stream);

/* Which kernel path BQ_PATH_AUTO takes for this shape (BQ_PATH_GEMV,
 * BQ_PATH_STREAM or BQ_PATH_TILED).  Host-only integer logic; no device call. */
int bq_gemm_select_path(int64_t M, int64_t N, int64_t K, int bits);

#ifdef __cplusplus
}
#endif

#endif /* BQ_H */
