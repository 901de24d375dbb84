// The C ABI of libqll.so: argument checks, workspace sizing and launches.
//
// Validation has one address -- here -- and the kernels below are unchecked
// and allocation-free (Fucina course "Chapter 06 -- Going fast on CPUs", 6.3
// "The kernel contract"; Fucina reference "Backends", 9.2).  Every check runs
// on the host before any HIP call, so an invalid call returns a status and
// never touches the device; an entry that cannot run says so instead of
// failing silently (the same reference, 9.9).
#include "../../include/qll.h"
#include "common.h"

#include <atomic>
#include <cstring>
#include <mutex>

using namespace qll;

// Scratch of qll_q4_0_q8_0_gemm_noalloc, for callers that cannot allocate:
// one array per device, held until the process ends.  In host code the name
// `scratch` only stands for the symbol; its device address on the current
// device comes from hipGetSymbolAddress (once per device, below), and only
// that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[QLL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;    // every dimension below 2^31
constexpr int64_t kMaxElems = (int64_t)1 << 40;  // and every tensor below 2^40 elements
constexpr int64_t kMaxGemmK = (int64_t)1 << 24;  // Q4_0/Q8_0 GEMMs (m > 8, repacked): 32-bit load offsets

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_ok(int64_t a, int64_t b)
{
    return a >= 1 && b >= 1 && a < kMaxDim && b < kMaxDim && a * b < kMaxElems;
}

// gfx950 check, once per device id (benign race: every writer stores the same).
std::atomic<int> g_arch_ok[64];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return QLL_ERR_DEVICE;
    if (dev < 64) {
        int v = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (v == 1)
            return QLL_OK;
        if (v == 2)
            return QLL_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return QLL_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64)
        g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? QLL_OK : QLL_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? QLL_OK : QLL_ERR_LAUNCH; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[64];

int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return QLL_ERR_DEVICE;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return QLL_ERR_DEVICE;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return QLL_OK;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

} // namespace

extern "C" {

const char *qll_status_string(int status)
{
    switch (status) {
    case QLL_OK:
        return "ok";
    case QLL_ERR_NULL:
        return "a required pointer is NULL";
    case QLL_ERR_SHAPE:
        return "invalid shape (size < 1, not a multiple of the block, or too large)";
    case QLL_ERR_ALIGN:
        return "a base address is not 16-byte aligned";
    case QLL_ERR_WORKSPACE:
        return "workspace missing or smaller than qll_workspace_bytes()";
    case QLL_ERR_LAUNCH:
        return "kernel launch failed";
    case QLL_ERR_DEVICE:
        return "no usable device or the current device is not gfx950";
    case QLL_ERR_SCRATCH:
        return "the shape needs more scratch than the allocation-free entry's static array holds";
    default:
        return "unknown status";
    }
}

size_t qll_workspace_bytes(int op, int64_t m, int64_t n, int64_t k)
{
    switch (op) {
    case QLL_OP_SGEMM:
        if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n))
            return SIZE_MAX;
        return m == 1 ? sgemv_workspace(n, k) : 0;
    case QLL_OP_Q4_0_Q8_0_GEMM:
        if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 32 != 0 || (m > kMaxMSmall && k >= kMaxGemmK))
            return SIZE_MAX;
        return q4_small_m_path(m, n, k) ? 0 : q4_0_q8_0_gemm_workspace(m, n, k);
    case QLL_OP_TERNARY_GEMM:
        if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 16 != 0)
            return SIZE_MAX;
        return 0;
    case QLL_OP_SGEMM_BF16:
        if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n))
            return SIZE_MAX;
        return gemm_nt_workspace(QLL_W_F32, m, n, k);
    case QLL_OP_GEMM_NT_BF16:
    case QLL_OP_GEMM_NT_F16:
    case QLL_OP_GEMM_NT_F32:
        if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n))
            return SIZE_MAX;
        return gemm_nt_workspace(op == QLL_OP_GEMM_NT_BF16 ? QLL_W_BF16 : op == QLL_OP_GEMM_NT_F16 ? QLL_W_F16 : QLL_W_F32,
                                 m, n, k);
    case QLL_OP_Q4_0_GEMV_F32:
        if (m < 1 || m > kMaxMSmall || !dims_ok(n, k) || k % 32 != 0)
            return SIZE_MAX;
        return q4_0_gemv_f32_workspace(m, n, k);
    case QLL_OP_Q4_0_REPACKED_GEMM:
    case QLL_OP_Q8_0_REPACKED_GEMM:
        if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 32 != 0 || k >= kMaxGemmK)
            return SIZE_MAX;
        return q4_0_packed_gemm_workspace(m, n, k);
    default:
        return SIZE_MAX;
    }
}

int qll_pack_q4_0(const uint8_t *codes, const uint16_t *d_bits, void *w, int64_t n, int64_t k, void *stream)
{
    if (!codes || !d_bits || !w)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(d_bits) || !aligned16(w))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_pack_q4_0(codes, d_bits, static_cast<uint8_t *>(w), n, k, as_stream(stream)));
}

int qll_pack_ternary(const uint8_t *codes, uint32_t *w, int64_t n, int64_t k, void *stream)
{
    if (!codes || !w)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 16 != 0)
        return QLL_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(w))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_pack_ternary(codes, w, n, k, as_stream(stream)));
}

int qll_quantize_q8_0(const float *x, void *xq, int64_t m, int64_t k, void *stream)
{
    if (!x || !xq)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(xq))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_quantize_q8_0(x, static_cast<uint8_t *>(xq), m * (k / 32), as_stream(stream)));
}

int qll_q4_0_q8_0_gemv(const void *w, const void *xq, float *y, int64_t n, int64_t k, void *stream)
{
    if (!w || !xq || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 32 != 0 || k > kMaxKQ4Gemv)
        return QLL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(xq) || !aligned16(y))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_q4_0_q8_0_gemv(static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(xq), y, n,
                                          k, as_stream(stream)));
}

int qll_q4_0_q8_0_gemv_f32(const void *w, const float *x, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                           size_t ws_bytes, void *stream)
{
    if (!w || !x || !y)
        return QLL_ERR_NULL;
    if (m < 1 || m > kMaxMSmall || !dims_ok(n, k) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    // a workspace too small, or not needed, selects the single launch
    const size_t need = q4_0_gemv_f32_workspace(m, n, k);
    uint8_t *wsp = (ws && need && ws_bytes >= need) ? static_cast<uint8_t *>(ws) : nullptr;
    if (!aligned16(w) || !aligned16(x) || !aligned16(y) || (wsp && !aligned16(wsp)))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(
        launch_q4_0_q8_0_gemv_f32(static_cast<const uint8_t *>(w), x, y, m, n, k, wsp, as_stream(stream)));
}

int qll_q4_0_q8_0_gemm(const void *w, const void *xq, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                       size_t ws_bytes, void *stream)
{
    if (!w || !xq || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    if (m == 1)
        return qll_q4_0_q8_0_gemv(w, xq, y, n, k, stream);
    if (!aligned16(w) || !aligned16(xq) || !aligned16(y))
        return QLL_ERR_ALIGN;
    if (q4_small_m_path(m, n, k)) {
        if (int rc = check_device())
            return rc;
        return launched(launch_q4_0_q8_0_gemv_m(static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(xq), y,
                                                m, n, k, as_stream(stream)));
    }
    if (k >= kMaxGemmK)
        return QLL_ERR_SHAPE;
    const size_t need = q4_0_q8_0_gemm_workspace(m, n, k);
    if (need > 0 && (!ws || ws_bytes < need))
        return QLL_ERR_WORKSPACE;
    if (ws && !aligned16(ws))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_q4_0_q8_0_gemm(static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(xq), y, m,
                                          n, k, ws, as_stream(stream)));
}

int qll_q4_0_q8_0_gemm_noalloc(const void *w, const void *xq, float *y, int64_t m, int64_t n, int64_t k,
                               void *stream)
{
    if (!w || !xq || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    if (q4_small_m_path(m, n, k)) // the small-m kernels need no scratch
        return qll_q4_0_q8_0_gemm(w, xq, y, m, n, k, nullptr, 0, stream);
    if (k >= kMaxGemmK)
        return QLL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(xq) || !aligned16(y))
        return QLL_ERR_ALIGN;
    if (q4_0_q8_0_gemm_workspace(m, n, k) > QLL_NOALLOC_SCRATCH_BYTES)
        return QLL_ERR_SCRATCH;
    if (int rc = check_device())
        return rc;
    void *ws = nullptr;
    if (int rc = scratch_address(&ws))
        return rc;
    return launched(launch_q4_0_q8_0_gemm(static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(xq), y, m,
                                          n, k, ws, as_stream(stream)));
}

size_t qll_q4_0_repacked_bytes(int64_t n, int64_t k)
{
    if (!dims_ok(n, k) || k % 32 != 0)
        return SIZE_MAX;
    return q4_0_repacked_bytes(n, k);
}

int qll_q4_0_repack(const void *w, void *wp, int64_t n, int64_t k, void *stream)
{
    if (!w || !wp)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(wp))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_q4_0_repack(static_cast<const uint8_t *>(w), static_cast<uint8_t *>(wp), n, k,
                                       as_stream(stream)));
}

size_t qll_q4_0_decode_packed_bytes(int64_t n, int64_t k)
{
    if (!dims_ok(n, k) || k % 32 != 0)
        return SIZE_MAX;
    return q4_0_packed_bytes(n, k);
}

int qll_q4_0_decode_pack(const void *w, void *wp, int64_t n, int64_t k, void *stream)
{
    if (!w || !wp)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(wp))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_q4_0_pack_decode(static_cast<const uint8_t *>(w), static_cast<uint8_t *>(wp), n, k,
                                            as_stream(stream)));
}

int qll_q4_0_decode_packed_q8_0_gemv(const void *wp, const void *xq, float *y, int64_t n, int64_t k, void *stream)
{
    if (!wp || !xq || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 32 != 0 || k > kMaxKQ4Gemv)
        return QLL_ERR_SHAPE;
    if (!aligned16(wp) || !aligned16(xq) || !aligned16(y))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_q4_0_packed_gemv(static_cast<const uint8_t *>(wp), static_cast<const uint8_t *>(xq), y, n,
                                            k, as_stream(stream)));
}

int qll_q4_0_repacked_q8_0_gemm(const void *wp, const void *xq, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                                size_t ws_bytes, void *stream)
{
    if (!wp || !xq || !y || !ws)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 32 != 0 || k >= kMaxGemmK)
        return QLL_ERR_SHAPE;
    if (!aligned16(wp) || !aligned16(xq) || !aligned16(y) || !aligned16(ws))
        return QLL_ERR_ALIGN;
    if (ws_bytes < q4_0_packed_gemm_workspace(m, n, k))
        return QLL_ERR_WORKSPACE;
    if (int rc = check_device())
        return rc;
    return launched(launch_q4_0_packed_gemm(static_cast<const uint8_t *>(wp), static_cast<const uint8_t *>(xq), y, m,
                                            n, k, ws, as_stream(stream)));
}

int qll_q8_0_q8_0_gemv(const void *w, const void *xq, float *y, int64_t n, int64_t k, void *stream)
{
    if (!w || !xq || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 32 != 0 || k > kMaxKQ4Gemv)
        return QLL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(xq) || !aligned16(y))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_q8_0_q8_0_gemv(static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(xq), y, n,
                                          k, as_stream(stream)));
}

size_t qll_q8_0_repacked_bytes(int64_t n, int64_t k)
{
    if (!dims_ok(n, k) || k % 32 != 0)
        return SIZE_MAX;
    return q8_0_repacked_bytes(n, k);
}

int qll_q8_0_repack(const void *w, void *wp, int64_t n, int64_t k, void *stream)
{
    if (!w || !wp)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 32 != 0)
        return QLL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(wp))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_q8_0_repack(static_cast<const uint8_t *>(w), static_cast<uint8_t *>(wp), n, k,
                                       as_stream(stream)));
}

int qll_q8_0_repacked_q8_0_gemm(const void *wp, const void *xq, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                                size_t ws_bytes, void *stream)
{
    if (!wp || !xq || !y || !ws)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 32 != 0 || k >= kMaxGemmK)
        return QLL_ERR_SHAPE;
    if (!aligned16(wp) || !aligned16(xq) || !aligned16(y) || !aligned16(ws))
        return QLL_ERR_ALIGN;
    if (ws_bytes < q4_0_packed_gemm_workspace(m, n, k))
        return QLL_ERR_WORKSPACE;
    if (int rc = check_device())
        return rc;
    return launched(launch_q8_0_packed_gemm(static_cast<const uint8_t *>(wp), static_cast<const uint8_t *>(xq), y, m,
                                            n, k, ws, as_stream(stream)));
}

int qll_gemm_nt(const float *x, const void *w, int w_dtype, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                size_t ws_bytes, void *stream)
{
    if (!x || !w || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || w_dtype < QLL_DTYPE_F32 || w_dtype > QLL_DTYPE_F16)
        return QLL_ERR_SHAPE;
    if (m > 1 && ((n + 127) / 128 > 0x7fffffff || (m + 127) / 128 > 65535))
        return QLL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (ws && !aligned16(ws)))
        return QLL_ERR_ALIGN;
    // bf16 weights at m > 1 always run on the bf16 matrix core and need the
    // workspace; f16 and f32 weights do when the workspace passed holds their
    // split parts, else they run (widened) on the f32 matrix core
    const bool core_shape = gemm_nt_bf16_core_shape(m, k);
    if (core_shape && w_dtype == QLL_DTYPE_BF16 && (!ws || ws_bytes < gemm_nt_workspace(w_dtype, m, n, k)))
        return QLL_ERR_WORKSPACE;
    const bool core = core_shape && ws != nullptr && ws_bytes >= gemm_nt_workspace(w_dtype, m, n, k);
    if (int rc = check_device())
        return rc;
    static_assert((int)QLL_DTYPE_F32 == (int)QLL_W_F32 && (int)QLL_DTYPE_BF16 == (int)QLL_W_BF16 &&
                      (int)QLL_DTYPE_F16 == (int)QLL_W_F16,
                  "dtype codes");
    if (m == 1)
        return launched(launch_gemv_nt(x, w, w_dtype, y, n, k, as_stream(stream)));
    if (core)
        return launched(launch_gemm_nt_bf16_mfma(x, w, w_dtype, y, m, n, k, ws, as_stream(stream)));
    return launched(launch_sgemm_nt(x, w, w_dtype, y, m, n, k, as_stream(stream)));
}

int qll_sgemm(const float *a, const float *b, float *c, int64_t m, int64_t n, int64_t k, void *ws, size_t ws_bytes,
              void *stream)
{
    if (!a || !b || !c)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n))
        return QLL_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(c))
        return QLL_ERR_ALIGN;
    if (m == 1) {
        const size_t need = sgemv_workspace(n, k);
        if (!ws || ws_bytes < need)
            return QLL_ERR_WORKSPACE;
        if (!aligned16(ws))
            return QLL_ERR_ALIGN;
        if (int rc = check_device())
            return rc;
        return launched(launch_sgemv(a, b, c, n, k, static_cast<float *>(ws), as_stream(stream)));
    }
    // m > 1: given a workspace that holds the split operands (and k % 16 ==
    // 0), on the bf16 matrix core with both operands split exactly into three
    // bf16 parts; otherwise on the f32 one
    const bool core = ws != nullptr && gemm_nt_bf16_core_shape(m, k) &&
                      ws_bytes >= gemm_nt_workspace(QLL_W_F32, m, n, k);
    if (core && !aligned16(ws))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    if (core)
        return launched(launch_gemm_nt_bf16_mfma(a, b, QLL_W_F32, c, m, n, k, ws, as_stream(stream), true));
    return launched(launch_sgemm(a, b, c, m, n, k, as_stream(stream)));
}

int qll_quantize_i8_rows(const float *x, int8_t *xq, float *act_scale, int32_t *act_sum, int64_t m, int64_t k,
                         void *stream)
{
    if (!x || !xq || !act_scale || !act_sum)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k))
        return QLL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(act_scale) || !aligned16(act_sum))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_quantize_i8_rows(x, xq, act_scale, act_sum, m, k, as_stream(stream)));
}

int qll_ternary_gemv(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                     const int32_t *act_sum, float *y, int64_t n, int64_t k, void *stream)
{
    if (!w || !xq || !act_scale || !act_sum || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(n, k) || k % 16 != 0 || k > kMaxKTernaryGemv)
        return QLL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(xq) || !aligned16(act_scale) || !aligned16(act_sum) || !aligned16(y))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_ternary_gemv(w, w_scale, xq, act_scale, act_sum, y, n, k, as_stream(stream)));
}

int qll_ternary_gemm(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                     const int32_t *act_sum, float *y, int64_t m, int64_t n, int64_t k, void *stream)
{
    if (!w || !xq || !act_scale || !act_sum || !y)
        return QLL_ERR_NULL;
    if (!dims_ok(m, k) || !dims_ok(n, k) || !dims_ok(m, n) || k % 16 != 0)
        return QLL_ERR_SHAPE;
    if (m == 1)
        return qll_ternary_gemv(w, w_scale, xq, act_scale, act_sum, y, n, k, stream);
    if (!aligned16(w) || !aligned16(xq) || !aligned16(act_scale) || !aligned16(act_sum) || !aligned16(y))
        return QLL_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return launched(launch_ternary_gemm(w, w_scale, xq, act_scale, act_sum, y, m, n, k, as_stream(stream)));
}

} // extern "C"
