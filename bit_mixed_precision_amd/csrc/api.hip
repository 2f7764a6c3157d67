// C ABI of libbq.so (declared in include/bq.h): host-side validation, the
// one-time device check, M-dispatch between the two GEMM kernels, launch.
//
// Validation follows the contracts of the pages' own entry points: BMINF's
// quantize() asserts dtypes and that the scale has the reduced shape, and
// its igemm asserts contiguity, device and matching K ("BMINF的後訓練量化實現",
// 實現代碼分析2); here each check returns a status instead of raising, and
// all checks run before anything is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/bq.h"
#include "bq_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return BQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return BQ_ERR_DEVICE;
    int st = g_device_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return BQ_ERR_HIP;
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? BQ_OK : BQ_ERR_DEVICE;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A launcher's grid check (kGridTooLarge) is a shape error; nothing was
// launched.  Any other failure is the runtime's.
int launch_status(hipError_t e)
{
    if (e == hipSuccess)
        return BQ_OK;
    return e == bq::kGridTooLarge ? BQ_ERR_SHAPE : BQ_ERR_HIP;
}

// Largest M handled by the streaming kernel (when asked for), and the largest
// M for which automatic dispatch takes it.  Below the MI355X ridge point
// (about 625 int8 operations per byte) the GEMM is bound by moving its
// operands; the streaming kernel loads A and B straight into matrix-core
// registers with K split over a workgroup's wavefronts, so its cost is the
// per-CU operand traffic (TM + TN bits/8) K of its tiles, while the tiled
// kernel stages tiles through LDS and reuses them across a larger tile.
// Measured (kernel trace, N = K = 4096): W4A8 M = 64 6.1 us streaming
// against 10.0 tiled, M = 128 7.8 against 10.4, M = 256 11.2 against 11.0;
// W8A8 M = 256 12.6 against 12.7; W2A8 M = 256 11.0 against 13.0.
constexpr int64_t kStreamMaxM = 256;
constexpr int64_t kStreamAutoMaxM = 128;
constexpr int64_t kStreamAutoMaxM2 = 256;  // int2 weights
// The dot-product GEMV accepts M <= 4 (each B byte feeds at most M
// multiply-adds); automatic dispatch uses it up to M = 2.
constexpr int64_t kGemvMaxM = 4;
constexpr int64_t kGemvAutoMaxM = 2;

int validate_gemm(const int8_t *A, const void *B, int bits, const void *scale, void *C,
                  int64_t M, int64_t N, int64_t K, int path)
{
    if (bits != 8 && bits != 4 && bits != 2)
        return BQ_ERR_ARG;
    if (path != BQ_PATH_AUTO && path != BQ_PATH_STREAM && path != BQ_PATH_TILED &&
        path != BQ_PATH_GEMV)
        return BQ_ERR_ARG;
    if (M < 0 || N < 0 || K < 0 || K > BQ_MAX_K || (K % 64) != 0)
        return BQ_ERR_SHAPE;
    if (M > BQ_MAX_DIM || N > BQ_MAX_DIM || M * N > BQ_MAX_OUT)
        return BQ_ERR_SHAPE;
    if (path == BQ_PATH_STREAM && M > kStreamMaxM)
        return BQ_ERR_SHAPE;
    if (path == BQ_PATH_GEMV && M > kGemvMaxM)
        return BQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return BQ_OK;
    if (!C || (K > 0 && (!A || !B)))
        return BQ_ERR_NULL;
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B))))
        return BQ_ERR_ALIGN;
    if (scale && !aligned16(scale))
        return BQ_ERR_ALIGN;
    return BQ_OK;
}

}  // namespace

extern "C" {

int bq_version(void) { return 100; }

const char *bq_status_string(int status)
{
    switch (status) {
    case BQ_OK: return "ok";
    case BQ_ERR_NULL: return "a required pointer is NULL";
    case BQ_ERR_SHAPE: return "invalid shape (negative dimension, divisibility or size limit)";
    case BQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case BQ_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case BQ_ERR_DEVICE: return "the current device is not gfx950";
    case BQ_ERR_ARG: return "invalid enumerated argument";
    default: return "unknown status";
    }
}

static int quantize_common(const void *x_f16, int64_t rows, int64_t cols, int qmax, int8_t *q,
                           void *scale_f16, void *stream)
{
    if (rows < 0 || cols < 0 || rows > INT32_MAX)
        return BQ_ERR_SHAPE;
    if (rows == 0)
        return BQ_OK;
    if (!scale_f16 || (cols > 0 && (!x_f16 || !q)))
        return BQ_ERR_NULL;
    if (!aligned16(scale_f16) || (cols > 0 && (!aligned16(x_f16) || !aligned16(q))))
        return BQ_ERR_ALIGN;
    const int dev = check_device();
    if (dev != BQ_OK)
        return dev;
    return launch_status(bq::launch_quantize_rows((const uint16_t *)x_f16, rows, cols, qmax, q,
                                                  (uint16_t *)scale_f16, (hipStream_t)stream));
}

int bq_quantize_rows(const void *x_f16, int64_t rows, int64_t cols, int8_t *q,
                     void *scale_f16, void *stream)
{
    return quantize_common(x_f16, rows, cols, 127, q, scale_f16, stream);
}

int bq_quantize_rows_bits(const void *x_f16, int64_t rows, int64_t cols, int bits, int8_t *q,
                          void *scale_f16, void *stream)
{
    if (bits != 8 && bits != 4 && bits != 2)
        return BQ_ERR_ARG;
    return quantize_common(x_f16, rows, cols, (1 << (bits - 1)) - 1, q, scale_f16, stream);
}

int bq_quantize_pack(const void *x_f16, int64_t rows, int64_t cols, int bits, uint8_t *packed,
                     void *scale_f16, void *stream)
{
    if (bits != 4 && bits != 2)
        return BQ_ERR_ARG;
    if (rows < 0 || cols < 0 || rows > INT32_MAX || (cols % (8 / bits)) != 0)
        return BQ_ERR_SHAPE;
    if (rows == 0)
        return BQ_OK;
    if (!scale_f16 || (cols > 0 && (!x_f16 || !packed)))
        return BQ_ERR_NULL;
    if (!aligned16(scale_f16) || (cols > 0 && (!aligned16(x_f16) || !aligned16(packed))))
        return BQ_ERR_ALIGN;
    const int dev = check_device();
    if (dev != BQ_OK)
        return dev;
    return launch_status(bq::launch_quantize_pack((const uint16_t *)x_f16, rows, cols, bits, packed,
                                                  (uint16_t *)scale_f16, (hipStream_t)stream));
}

static int pack_common(const int8_t *v, int64_t n, int64_t k, uint8_t *out, int factor)
{
    if (n < 0 || k < 0 || (k % factor) != 0)
        return BQ_ERR_SHAPE;
    if (n == 0 || k == 0)
        return BQ_OK;
    if (!v || !out)
        return BQ_ERR_NULL;
    if (!aligned16(v) || !aligned16(out))
        return BQ_ERR_ALIGN;
    return check_device();
}

int bq_pack_int4(const int8_t *v, int64_t n, int64_t k, uint8_t *out, void *stream)
{
    const int st = pack_common(v, n, k, out, 2);
    if (st != BQ_OK || n == 0 || k == 0)
        return st;
    return launch_status(bq::launch_pack_int4(v, n * k, out, (hipStream_t)stream));
}

int bq_pack_int2(const int8_t *v, int64_t n, int64_t k, uint8_t *out, void *stream)
{
    const int st = pack_common(v, n, k, out, 4);
    if (st != BQ_OK || n == 0 || k == 0)
        return st;
    return launch_status(bq::launch_pack_int2(v, n * k, out, (hipStream_t)stream));
}

int bq_gemm_select_path(int64_t M, int64_t N, int64_t K, int bits)
{
    (void)N;
    (void)K;
    if (M <= kGemvAutoMaxM)
        return BQ_PATH_GEMV;
    return M <= (bits == 2 ? kStreamAutoMaxM2 : kStreamAutoMaxM) ? BQ_PATH_STREAM : BQ_PATH_TILED;
}

static int gemm_common(const int8_t *A, const void *B, int bits, const void *scale_f16,
                       const void *xscale_f16, int act, void *C, int64_t M, int64_t N, int64_t K,
                       int path, void *stream, int batch = 1, const bq::BatchStrides &bs = {},
                       void *ws = nullptr, int64_t wsBytes = 0)
{
    int st = validate_gemm(A, B, bits, scale_f16, C, M, N, K, path);
    if (st != BQ_OK || M == 0 || N == 0)
        return st;
    st = check_device();
    if (st != BQ_OK)
        return st;
    if (path == BQ_PATH_AUTO)
        path = bq_gemm_select_path(M, N, K, bits);
    const hipStream_t s = (hipStream_t)stream;
    const uint8_t *Bb = (const uint8_t *)B;
    const uint16_t *sc = (const uint16_t *)scale_f16;
    const uint16_t *xs = (const uint16_t *)xscale_f16;
    if (path == BQ_PATH_GEMV)
        return launch_status(bq::launch_gemv(A, Bb, bits, sc, xs, act, C, (int)M, (int)N, (int)K, batch, bs, s));
    if (path == BQ_PATH_STREAM)
        return launch_status(bq::launch_gemm_stream(A, Bb, bits, sc, xs, act, C, (int)M, (int)N, (int)K, batch, bs, s));
    return launch_status(
        bq::launch_gemm_tiled(A, Bb, bits, sc, xs, act, C, (int)M, (int)N, (int)K, batch, bs, s, ws, wsBytes));
}

int bq_gemm(const int8_t *A, const void *B, int bits, const void *scale_f16, void *C,
            int64_t M, int64_t N, int64_t K, int path, void *stream)
{
    return gemm_common(A, B, bits, scale_f16, nullptr, 0, C, M, N, K, path, stream);
}

int64_t bq_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits)
{
    if (bits != 8 && bits != 4 && bits != 2)
        return -BQ_ERR_ARG;
    if (M < 0 || N < 0 || K < 0 || K > BQ_MAX_K || (K % 64) != 0 || M > BQ_MAX_DIM || N > BQ_MAX_DIM ||
        M * N > BQ_MAX_OUT)
        return -BQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return 0;
    return bq::gemm_splitk_workspace_bytes((int)M, (int)N, (int)K, bits);
}

int bq_gemm_splitk(const int8_t *A, const void *B, int bits, const void *scale_f16, void *C, int64_t M,
                   int64_t N, int64_t K, void *workspace, int64_t workspace_bytes, void *stream)
{
    if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
        return workspace_bytes < 0 ? BQ_ERR_SHAPE : BQ_ERR_NULL;
    if (workspace && !aligned16(workspace))
        return BQ_ERR_ALIGN;
    return gemm_common(A, B, bits, scale_f16, nullptr, 0, C, M, N, K, BQ_PATH_TILED, stream, 1, {},
                       workspace_bytes > 0 ? workspace : nullptr, workspace_bytes);
}

// ---- allocation-free split-K (bq_gemm_splitk_static) ----

// Bytes of the library's own split-K scratch: the largest workspace any
// shape asks for (4 KiB of per-tile counters, 16 KiB of partial sums for
// each of at most 256 workgroups).
constexpr int64_t kScratchBytes = 4096 + 256 * 16384;

}  // extern "C"

// The scratch memory of bq_gemm_splitk_static: one copy on every GPU the
// library runs on, zero when the code object is loaded, held until the
// process ends.  In host code `scratch` is not a device address; the kernels
// receive the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return BQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return BQ_ERR_DEVICE;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return BQ_ERR_HIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BQ_OK;
}

// Zero n 32-bit words (a kernel, not a memset, so that a captured graph
// replays it as a kernel node).
__global__ void zero_words_kernel(int *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0;
}

}  // namespace

extern "C" {

int bq_gemm_splitk_static(const int8_t *A, const void *B, int bits, const void *scale_f16, void *C, int64_t M,
                          int64_t N, int64_t K, void *stream)
{
    int st = validate_gemm(A, B, bits, scale_f16, C, M, N, K, BQ_PATH_TILED);
    if (st != BQ_OK || M == 0 || N == 0)
        return st;
    const int64_t need = bq::gemm_splitk_workspace_bytes((int)M, (int)N, (int)K, bits);
    if (need > kScratchBytes)
        return BQ_ERR_SHAPE;
    st = check_device();
    if (st != BQ_OK)
        return st;
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_address(&ws);
        if (st != BQ_OK)
            return st;
        // the per-tile counters start at zero whatever an earlier call left
        constexpr int kCtrWords = 4096 / 4;
        zero_words_kernel<<<kCtrWords / 256, 256, 0, (hipStream_t)stream>>>((int *)ws, kCtrWords);
        st = launch_status(hipGetLastError());
        if (st != BQ_OK)
            return st;
    }
    return gemm_common(A, B, bits, scale_f16, nullptr, 0, C, M, N, K, BQ_PATH_TILED, stream, 1, {}, ws,
                       ws ? kScratchBytes : 0);
}

// Largest batch of bq_gemm_batched (the grid's y dimension).
constexpr int64_t kMaxBatch = 65535;

int bq_gemm_batched(const int8_t *A, int64_t strideA, const void *B, int64_t strideB, int bits,
                    const void *scale_f16, int64_t strideScale, const void *x_scale_f16,
                    void *C, int64_t strideC, int64_t batch, int64_t M, int64_t N, int64_t K,
                    int path, void *stream)
{
    if (batch < 0 || batch > kMaxBatch || strideA < 0 || strideB < 0 || strideScale < 0 || strideC < 0 ||
        M < 0 || N < 0)
        return BQ_ERR_SHAPE;
    // an empty batch is a no-op like M = 0 or N = 0 (arguments other than
    // pointers still checked)
    int st = validate_gemm(A, B, bits, scale_f16, C, batch == 0 ? 0 : M, N, K, path);
    if (st != BQ_OK || batch == 0 || M == 0 || N == 0)
        return st;
    // outputs of different batches must not overlap; inputs may (stride 0
    // broadcasts one operand to every batch)
    if (batch > 1 && strideC < M * N)
        return BQ_ERR_SHAPE;
    if (x_scale_f16 && !scale_f16)
        return BQ_ERR_NULL;
    if (x_scale_f16 && !aligned16(x_scale_f16))
        return BQ_ERR_ALIGN;
    // every batch's operands start 16-byte aligned
    const int64_t outBytes = scale_f16 ? 2 : 4;
    if ((strideA % 16) != 0 || (strideB % 16) != 0 || ((strideScale * 2) % 16) != 0 ||
        ((strideC * outBytes) % 16) != 0)
        return BQ_ERR_ALIGN;
    bq::BatchStrides bs;
    bs.a = strideA;
    bs.b = strideB;
    bs.s = strideScale;
    bs.c = strideC;
    return gemm_common(A, B, bits, scale_f16, x_scale_f16, 0, C, M, N, K, path, stream, (int)batch, bs);
}

int bq_gemm_dual_scale(const int8_t *A, const void *B, int bits, const void *w_scale_f16,
                       const void *x_scale_f16, void *C_f16, int64_t M, int64_t N, int64_t K,
                       int path, void *stream)
{
    if (M > 0 && N > 0 && (!w_scale_f16 || !x_scale_f16))
        return BQ_ERR_NULL;
    if (x_scale_f16 && !aligned16(x_scale_f16))
        return BQ_ERR_ALIGN;
    return gemm_common(A, B, bits, w_scale_f16, x_scale_f16, 0, C_f16, M, N, K, path, stream);
}

int bq_gemm_act(const int8_t *A, const void *B, int bits, const void *w_scale_f16,
                const void *x_scale_f16, int act, void *C_f16, int64_t M, int64_t N, int64_t K,
                int path, void *stream)
{
    if (act != BQ_ACT_NONE && act != BQ_ACT_RELU && act != BQ_ACT_GELU)
        return BQ_ERR_ARG;
    if (M > 0 && N > 0 && !w_scale_f16)
        return BQ_ERR_NULL;
    if (x_scale_f16 && !aligned16(x_scale_f16))
        return BQ_ERR_ALIGN;
    return gemm_common(A, B, bits, w_scale_f16, x_scale_f16, act, C_f16, M, N, K, path, stream);
}

int bq_gemm_nf4_a16(const void *A_f16, const uint8_t *B, const void *scale_f16, const void *zero_f16,
                    void *C_f16, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (M < 0 || N < 0 || K < 0 || K > BQ_MAX_K || (K % 64) != 0 || M > BQ_MAX_DIM || N > BQ_MAX_DIM ||
        M * N > BQ_MAX_OUT)
        return BQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return BQ_OK;
    if (!C_f16 || !scale_f16 || (K > 0 && (!A_f16 || !B)))
        return BQ_ERR_NULL;
    if (!aligned16(C_f16) || !aligned16(scale_f16) || (zero_f16 && !aligned16(zero_f16)) ||
        (K > 0 && (!aligned16(A_f16) || !aligned16(B))))
        return BQ_ERR_ALIGN;
    const int st = check_device();
    if (st != BQ_OK)
        return st;
    if (M <= kGemvMaxM)
        return launch_status(bq::launch_gemv_nf4((const uint16_t *)A_f16, B, (const uint16_t *)scale_f16,
                                                 (const uint16_t *)zero_f16, (uint16_t *)C_f16, (int)M, (int)N,
                                                 (int)K, (hipStream_t)stream));
    return launch_status(bq::launch_gemm_nf4((const uint16_t *)A_f16, B, (const uint16_t *)scale_f16,
                                             (const uint16_t *)zero_f16, (uint16_t *)C_f16, (int)M, (int)N,
                                             (int)K, (hipStream_t)stream));
}

int bq_gemm_w8a8_dequant(const int8_t *A, const int8_t *B, const void *scale_f16,
                         void *C_f16, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (!scale_f16 && M > 0 && N > 0)
        return BQ_ERR_NULL;
    return bq_gemm(A, B, 8, scale_f16, C_f16, M, N, K, BQ_PATH_AUTO, stream);
}

int bq_gemm_w4a8_dequant(const int8_t *A, const uint8_t *B, const void *scale_f16,
                         void *C_f16, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (!scale_f16 && M > 0 && N > 0)
        return BQ_ERR_NULL;
    return bq_gemm(A, B, 4, scale_f16, C_f16, M, N, K, BQ_PATH_AUTO, stream);
}

int bq_gemm_w2a8_dequant(const int8_t *A, const uint8_t *B, const void *scale_f16,
                         void *C_f16, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (!scale_f16 && M > 0 && N > 0)
        return BQ_ERR_NULL;
    return bq_gemm(A, B, 2, scale_f16, C_f16, M, N, K, BQ_PATH_AUTO, stream);
}

int bq_gemm_w8a8_i32(const int8_t *A, const int8_t *B, int32_t *C_i32,
                     int64_t M, int64_t N, int64_t K, void *stream)
{
    return bq_gemm(A, B, 8, nullptr, C_i32, M, N, K, BQ_PATH_AUTO, stream);
}

int bq_gemm_w4a8_i32(const int8_t *A, const uint8_t *B, int32_t *C_i32,
                     int64_t M, int64_t N, int64_t K, void *stream)
{
    return bq_gemm(A, B, 4, nullptr, C_i32, M, N, K, BQ_PATH_AUTO, stream);
}

int bq_gemm_w2a8_i32(const int8_t *A, const uint8_t *B, int32_t *C_i32,
                     int64_t M, int64_t N, int64_t K, void *stream)
{
    return bq_gemm(A, B, 2, nullptr, C_i32, M, N, K, BQ_PATH_AUTO, stream);
}

}  // extern "C"
