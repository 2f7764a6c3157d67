/*
 * bqref.c - the oracle: a plain, slow, obviously correct CPU implementation
 * of the quantize -> pack -> integer GEMM -> fp16 dequant path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the HIP
 * kernels.
 *
 * Floating point is done in IEEE double with the default round-to-nearest-even
 * mode; fp16 values travel as their 16-bit patterns and are decoded/encoded
 * by the codec below, written from the IEEE 754 binary16 definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits, subnormals,
 * infinities, NaN).
 *
 * Sources for what is computed (cited by page title and section):
 *  - "BMINF的後訓練量化實現" (BMINF post-training quantization), section
 *    實現代碼分析2, the quantize() docstring of PartialAttention.quantize:
 *    per-row absolute maximum divided by 127 as an fp16 scale (reduction
 *    kernel bms_quantize_scale), codes = nearest integer of x / scale
 *    (elementwise kernel bms_quantize_copy_*), symmetric, no zero point;
 *    the quantized weight parameter layout (int8 [out, in] with an fp16
 *    scale of shape [out, 1]) in the PartialAttention constructor.
 *  - "BitBLAS自定义操作开发指南：使用DSL扩展新的混合精度算子" (BitBLAS
 *    custom-operator guide), sections 1 (create_mixed_precision_matmul:
 *    C[i,j] = sum_k int32(A[i,k]) * int32(B[j,k]), A int8 [M,K], B [N,K]),
 *    2 (create_dequantize_matmul: the int32 result times scale[j]),
 *    case 1 (BitNet-b1.58 int2 weights), case 2 (sub-byte weights stored
 *    compressed as uint8 [N, K/2]).
 *
 * Status codes: 0 ok, 1 null pointer, 2 bad shape, 3 value out of range
 * (non-finite input, pack value outside the code range, int32 overflow).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define BQREF_OK 0
#define BQREF_ERR_NULL 1
#define BQREF_ERR_SHAPE 2
#define BQREF_ERR_RANGE 3

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 codec                                                   */
/* ------------------------------------------------------------------------ */

/* binary16 bit pattern -> exact double. */
double bqref_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1.frac) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* double -> binary16 bit pattern, rounded to nearest, ties to even.
 * Magnitudes at or above 65520 (the midpoint between the largest finite
 * value 65504 and 2^16) round to infinity. */
uint16_t bqref_f64_to_f16(double d)
{
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    double a = fabs(d);
    if (isnan(d))
        return 0x7e00;
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: a multiple of the quantum 2^-24; n may round up to
         * 1024, which is exactly the bit pattern of the smallest normal. */
        double n = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)n;
    }
    int e2;
    frexp(a, &e2);           /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;          /* a in [2^e, 2^(e+1)), e in [-14, 15] */
    double n = nearbyint(ldexp(a, 10 - e)); /* significand in [1024, 2048] */
    /* n == 2048 carries into the exponent field by plain addition. */
    return sign | (uint16_t)(((e + 15) << 10) + (int)(n - 1024.0));
}

void bqref_f16_to_f64_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bqref_f16_to_f64(h[i]);
}

void bqref_f64_to_f16_array(const double *d, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bqref_f64_to_f16(d[i]);
}

/* ------------------------------------------------------------------------ */
/* Step 1+2: per-row symmetric int8 quantization (BMINF page)               */
/* ------------------------------------------------------------------------ */

/* For each row r of x [rows, cols] (fp16, row-major) and a code range
 * qmax (127 for int8 as on the BMINF page; 7 and 1 give the int4 and
 * ternary code ranges, qmax = 2^(bits-1) - 1):
 *   amax_r  = max_k |x[r,k]|                      (exact)
 *   scale_r = fp16 nearest to amax_r / qmax        (ties to even)
 *   q[r,k]  = nearest integer to x[r,k] / scale_r  (ties to even),
 *             clamped to [-qmax, qmax]
 * A row whose scale rounds to zero (all zeros, or amax at most 63 * 2^-24)
 * gets scale 0 and codes 0.
 *
 * Exactness of the double arithmetic used here: amax/qmax and x/scale are
 * quotients of fp16 values; neither can fall within double precision of a
 * rounding midpoint of the target format (fp16 resp. the half-integers)
 * without being exactly on it, because both operands carry at most 11
 * significant bits while the target grid is at least 2^-13 relative apart
 * from any such quotient; so rounding the double quotient once more gives
 * the correctly rounded result of the exact quotient. */
int bqref_quantize_rows_q(const uint16_t *x, int64_t rows, int64_t cols, int qmax,
                          int8_t *q, uint16_t *scale)
{
    if (rows < 0 || cols < 0)
        return BQREF_ERR_SHAPE;
    if (qmax < 1 || qmax > 127)
        return BQREF_ERR_RANGE;
    if (rows > 0 && (!scale || (cols > 0 && (!x || !q))))
        return BQREF_ERR_NULL;
    int status = BQREF_OK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * cols;
        double amax = 0.0;
        int bad = 0;
        for (int64_t k = 0; k < cols; ++k) {
            double v = bqref_f16_to_f64(xr[k]);
            if (!isfinite(v))
                bad = 1;
            else if (fabs(v) > amax)
                amax = fabs(v);
        }
        if (bad) {
#pragma omp atomic write
            status = BQREF_ERR_RANGE;
            continue;
        }
        uint16_t s16 = bqref_f64_to_f16(amax / (double)qmax);
        double s = bqref_f16_to_f64(s16);
        scale[r] = s16;
        for (int64_t k = 0; k < cols; ++k) {
            double c = 0.0;
            if (s != 0.0) {
                c = nearbyint(bqref_f16_to_f64(xr[k]) / s);
                if (c > qmax)
                    c = qmax;
                if (c < -qmax)
                    c = -qmax;
            }
            q[r * cols + k] = (int8_t)c;
        }
    }
    return status;
}

/* The int8 form of the BMINF page (qmax = 127). */
int bqref_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols,
                        int8_t *q, uint16_t *scale)
{
    return bqref_quantize_rows_q(x, rows, cols, 127, q, scale);
}

/* ------------------------------------------------------------------------ */
/* Step 3: packing of sub-byte weights along K                              */
/* ------------------------------------------------------------------------ */

/* int4: byte [n, k/2] holds v[n,k] in its low nibble and v[n,k+1] in its high
 * nibble (k even), each as a 4-bit two's complement number in [-8, 7]. */
int bqref_pack_int4(const int8_t *v, int64_t n, int64_t k, uint8_t *out)
{
    if (n < 0 || k < 0 || (k % 2) != 0)
        return BQREF_ERR_SHAPE;
    if (n * k > 0 && (!v || !out))
        return BQREF_ERR_NULL;
    for (int64_t i = 0; i < n * k; ++i)
        if (v[i] < -8 || v[i] > 7)
            return BQREF_ERR_RANGE;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k / 2; ++j) {
            int lo = v[r * k + 2 * j];
            int hi = v[r * k + 2 * j + 1];
            out[r * (k / 2) + j] = (uint8_t)(((unsigned)lo & 0xF) | (((unsigned)hi & 0xF) << 4));
        }
    return BQREF_OK;
}

int bqref_unpack_int4(const uint8_t *p, int64_t n, int64_t k, int8_t *v)
{
    if (n < 0 || k < 0 || (k % 2) != 0)
        return BQREF_ERR_SHAPE;
    if (n * k > 0 && (!v || !p))
        return BQREF_ERR_NULL;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j) {
            uint8_t byte = p[r * (k / 2) + j / 2];
            int nib = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            v[r * k + j] = (int8_t)(nib >= 8 ? nib - 16 : nib);
        }
    return BQREF_OK;
}

/* int2 (BitNet-b1.58 ternary weights): byte [n, k/4] holds the 2-bit code
 * v+2 of v[n, k+j] in bits 2j..2j+1 (k a multiple of 4, j = 0..3), so the
 * lowest bits hold the lowest k.  Codes 0..3 represent -2..1; ternary data
 * uses -1, 0, 1 only. */
int bqref_pack_int2(const int8_t *v, int64_t n, int64_t k, uint8_t *out)
{
    if (n < 0 || k < 0 || (k % 4) != 0)
        return BQREF_ERR_SHAPE;
    if (n * k > 0 && (!v || !out))
        return BQREF_ERR_NULL;
    for (int64_t i = 0; i < n * k; ++i)
        if (v[i] < -2 || v[i] > 1)
            return BQREF_ERR_RANGE;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 4; ++b) {
            unsigned byte = 0;
            for (int j = 0; j < 4; ++j)
                byte |= (unsigned)(v[r * k + 4 * b + j] + 2) << (2 * j);
            out[r * (k / 4) + b] = (uint8_t)byte;
        }
    return BQREF_OK;
}

int bqref_unpack_int2(const uint8_t *p, int64_t n, int64_t k, int8_t *v)
{
    if (n < 0 || k < 0 || (k % 4) != 0)
        return BQREF_ERR_SHAPE;
    if (n * k > 0 && (!v || !p))
        return BQREF_ERR_NULL;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j) {
            uint8_t byte = p[r * (k / 4) + j / 4];
            int code = (byte >> (2 * (j % 4))) & 3;
            v[r * k + j] = (int8_t)(code - 2);
        }
    return BQREF_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 4: integer GEMM with int32 result (BitBLAS page, section 1)          */
/* ------------------------------------------------------------------------ */

/* C[m,n] = sum_k A[m,k] * B[n,k]; A int8 [M,K], B int8 values [N,K] (already
 * unpacked), C int32 [M,N]; all row-major.  The sum is formed exactly in
 * 64-bit integers and must fit in int32 (otherwise ERR_RANGE: the method
 * accumulates in int32). */
int bqref_gemm_i32(const int8_t *A, const int8_t *B, int32_t *C,
                   int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0)
        return BQREF_ERR_SHAPE;
    if (M * N > 0 && (!C || (K > 0 && (!A || !B))))
        return BQREF_ERR_NULL;
    int status = BQREF_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
            if (acc > INT32_MAX || acc < INT32_MIN) {
#pragma omp atomic write
                status = BQREF_ERR_RANGE;
            }
            C[m * N + n] = (int32_t)acc;
        }
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* Step 5: dequant epilogue (BitBLAS page, section 2)                        */
/* ------------------------------------------------------------------------ */

/* out[m,n] = fp16 nearest to acc[m,n] * scale[n] (ties to even; overflow to
 * +-inf).  The double product of an int32 and an fp16 value is exact, so
 * this is one correct rounding of the real product. */
int bqref_dequant(const int32_t *acc, const uint16_t *scale, uint16_t *out,
                  int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return BQREF_ERR_SHAPE;
    if (M * N > 0 && (!acc || !scale || !out))
        return BQREF_ERR_NULL;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = bqref_f64_to_f16((double)acc[m * N + n] * bqref_f16_to_f64(scale[n]));
    return BQREF_OK;
}

/* ------------------------------------------------------------------------ */
/* Two-scale dequant of a linear layer with per-token activation scales     */
/* (BMINF page, section 實現代碼分析2, PartialAttention forward: the input is */
/* quantized per token with quantize(..., axis=1), multiplied by the int8    */
/* weight with igemm, and each int32 result is multiplied by the scale of    */
/* its output channel and the scale of its token, out0 = in0 * in1 * in2)   */
/* ------------------------------------------------------------------------ */

/* out[m,n] = fp16 nearest to acc[m,n] * w_scale[n] * x_scale[m] (ties to
 * even; overflow to +-inf).  The double product is exact: |acc| < 2^31 and
 * the two fp16 significands have 11 bits each, 31 + 11 + 11 = 53, so this is
 * one correct rounding of the real product. */
int bqref_dequant2(const int32_t *acc, const uint16_t *w_scale, const uint16_t *x_scale,
                   uint16_t *out, int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return BQREF_ERR_SHAPE;
    if (M * N > 0 && (!acc || !w_scale || !x_scale || !out))
        return BQREF_ERR_NULL;
    for (int64_t m = 0; m < M; ++m) {
        const double xs = bqref_f16_to_f64(x_scale[m]);
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = bqref_f64_to_f16((double)acc[m * N + n] * bqref_f16_to_f64(w_scale[n]) * xs);
    }
    return BQREF_OK;
}

/* ------------------------------------------------------------------------ */
/* Activation fused into the epilogue (JAX Pallas matmul page, fused-        */
/* activation section: the activation is applied once, to the wide           */
/* accumulated result of the last K step, before the single downcast;       */
/* BladeDISC page, CUTLASS GEMM codegen: GEMM followed by GELU fused)       */
/* ------------------------------------------------------------------------ */

/* act 0: identity; 1: ReLU max(v, 0); 2: GELU v * Phi(v) with the standard
 * normal CDF Phi(v) = erfc(-v / sqrt(2)) / 2 (the complementary form has no
 * cancellation for negative v). */
double bqref_act(double v, int act)
{
    if (act == 1)
        return v > 0.0 ? v : 0.0;
    if (act == 2)
        return 0.5 * v * erfc(-v / sqrt(2.0));
    return v;
}

/* out[m,n] = fp16 nearest to act(acc[m,n] * w_scale[n] * x_scale[m]) with
 * x_scale NULL meaning 1.  The product is exact in double (see dequant2);
 * ReLU keeps it exact; GELU is evaluated in double (libm erfc) and rounded
 * once to fp16. */
int bqref_dequant_act(const int32_t *acc, const uint16_t *w_scale, const uint16_t *x_scale,
                      int act, uint16_t *out, int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return BQREF_ERR_SHAPE;
    if (act < 0 || act > 2)
        return BQREF_ERR_RANGE;
    if (M * N > 0 && (!acc || !w_scale || !out))
        return BQREF_ERR_NULL;
    for (int64_t m = 0; m < M; ++m) {
        const double xs = x_scale ? bqref_f16_to_f64(x_scale[m]) : 1.0;
        for (int64_t n = 0; n < N; ++n) {
            const double v = (double)acc[m * N + n] * bqref_f16_to_f64(w_scale[n]) * xs;
            out[m * N + n] = bqref_f64_to_f16(bqref_act(v, act));
        }
    }
    return BQREF_OK;
}
