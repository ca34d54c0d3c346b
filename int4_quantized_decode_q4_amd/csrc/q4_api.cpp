// q4_api.cpp -- the extern "C" entry points of libq4 (declared in
// include/q4.h): host-side validation, then one launch on the caller's
// stream.  Validation never touches the HIP runtime, so every error path can
// be exercised on a machine without a GPU.
#include <stdint.h>
#include <atomic>
#include <cmath>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/q4.h"
#include "q4_geometry.h"
#include "q4_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // 0 = not asked yet

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Do [a, a + an) and [b, b + bn) share a byte?
bool overlap(const void *a, int64_t an, const void *b, int64_t bn)
{
    if (!a || !b || an <= 0 || bn <= 0)
        return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)bn && pb < pa + (uintptr_t)an;
}

bool valid_shape(int64_t n, int64_t k)
{
    // sizes stay far inside int64 (n, k < 2^31); the GEMV family indexes rows
    // as int32 in its argmax, so a layout must have fewer than 2^31 rows.
    return n >= 1 && k >= 32 && (k % 32) == 0 && n <= (int64_t)INT32_MAX / 2;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return Q4_OK;
    g_last_hip_error = (int)e;
    return Q4_ERR_HIP;
}

// Checks shared by every op that reads a packed weight; returns the logical
// row count of the layout through `rows`.
int check_weight(const q4_weight *w, int32_t want_layout, q4::Geometry *geo, int64_t *rows)
{
    if (!w || !w->data)
        return Q4_ERR_NULL;
    if (!valid_shape(w->n, w->k))
        return Q4_ERR_SHAPE;
    if (w->layout != want_layout || w->version != Q4_LAYOUT_VERSION)
        return Q4_ERR_LAYOUT;
    if (!aligned(w->data, 256))
        return Q4_ERR_ALIGN;
    if (w->layout == Q4_LAYOUT_ROPE &&
        (w->head_dim < 2 || w->head_dim % 2 != 0 || w->n % w->head_dim != 0))
        return Q4_ERR_SHAPE;
    const bool int3 = w->layout == Q4_LAYOUT_INT3 || w->layout == Q4_LAYOUT_INT3_GATE_UP;
    *rows = (want_layout == Q4_LAYOUT_GATE_UP || want_layout == Q4_LAYOUT_INT3_GATE_UP)
                ? 2 * (int64_t)w->n
                : (int64_t)w->n;
    const bool ok = int3 ? q4::layout_geometry3(*rows, w->k, geo)
                         : q4::layout_geometry(*rows, w->k, geo);
    if (!ok)
        return Q4_ERR_SHAPE;
    if (w->bytes < geo->tiles * geo->tile_bytes)
        return Q4_ERR_SIZE;
    return Q4_OK;
}

int pack_common(const uint32_t *w0, const uint16_t *s0, const uint32_t *w1, const uint16_t *s1,
                int32_t n, int32_t k, q4::PackMode mode, int32_t d, void *dst, int64_t dst_bytes,
                q4_weight *out, void *stream)
{
    const bool gate_up = mode == q4::PACK_GATE_UP;
    if (!w0 || !s0 || !dst || !out || (gate_up && (!w1 || !s1)))
        return Q4_ERR_NULL;
    if (!valid_shape(n, k))
        return Q4_ERR_SHAPE;
    if (mode == q4::PACK_ROPE && (d < 2 || d % 2 != 0 || n % d != 0))
        return Q4_ERR_SHAPE;
    if (!aligned(w0, 16) || !aligned(s0, 2) || !aligned(dst, 256) ||
        (gate_up && (!aligned(w1, 16) || !aligned(s1, 2))))
        return Q4_ERR_ALIGN;
    const int64_t rows = gate_up ? 2 * (int64_t)n : (int64_t)n;
    q4::Geometry geo;
    if (!q4::layout_geometry(rows, k, &geo))
        return Q4_ERR_SHAPE;
    const int64_t need = geo.tiles * geo.tile_bytes;
    if (dst_bytes < need)
        return Q4_ERR_SIZE;
    const int64_t wbytes = (int64_t)n * k / 2, sbytes = (int64_t)n * (k / 32) * 2;
    if (overlap(dst, need, w0, wbytes) || overlap(dst, need, s0, sbytes) ||
        (gate_up && (overlap(dst, need, w1, wbytes) || overlap(dst, need, s1, sbytes))))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    const int rc = hip_status(q4::launch_pack(w0, s0, w1, s1, rows, k, mode, d, geo, dst,
                                              static_cast<hipStream_t>(stream)));
    if (rc != Q4_OK)
        return rc;
    out->n = n;
    out->k = k;
    out->layout = gate_up ? Q4_LAYOUT_GATE_UP
                          : (mode == q4::PACK_ROPE ? Q4_LAYOUT_ROPE : Q4_LAYOUT_ROWS);
    out->version = Q4_LAYOUT_VERSION;
    out->data = dst;
    out->bytes = need;
    out->head_dim = mode == q4::PACK_ROPE ? d : 0;
    out->reserved = 0;
    return Q4_OK;
}

}  // namespace

// ------------------------------------------------------- static scratch --
// The scratch of the allocation-free entry point (q4_lmhead_f32_noalloc):
// one file-scope device array, present on every GPU the library runs on
// for the life of the process.  Host code never uses the array's name as an
// address (on the host it is only a stand-in symbol): its device address is
// asked for once per device with hipGetSymbolAddress, and that pointer is
// what the kernels get.
namespace {
constexpr int64_t kNoAllocScratchBytes = 64 * 1024;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::atomic<void *> g_scratch[kMaxDevices];

// The current device's address of `scratch` (nullptr and *rc = the error on
// failure).
void *noalloc_scratch(int *rc)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *rc = hip_status(e != hipSuccess ? e : hipErrorInvalidDevice);
        return nullptr;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            *rc = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return nullptr;
        }
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}
}  // namespace

int q4::device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) {
            (void)hipGetLastError();
            c = 256;
        }
        g_cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

extern "C" {

int64_t q4_packed_bytes(int32_t n, int32_t k, int32_t layout)
{
    if (!valid_shape(n, k) ||
        (layout != Q4_LAYOUT_ROWS && layout != Q4_LAYOUT_GATE_UP && layout != Q4_LAYOUT_ROPE &&
         layout != Q4_LAYOUT_INT3 && layout != Q4_LAYOUT_INT3_GATE_UP))
        return 0;
    q4::Geometry geo;
    const int64_t rows = (layout == Q4_LAYOUT_GATE_UP || layout == Q4_LAYOUT_INT3_GATE_UP)
                             ? 2 * (int64_t)n
                             : (int64_t)n;
    if (layout == Q4_LAYOUT_INT3 || layout == Q4_LAYOUT_INT3_GATE_UP)
        return q4::layout_geometry3(rows, k, &geo) ? geo.tiles * geo.tile_bytes : 0;
    if (!q4::layout_geometry(rows, k, &geo))
        return 0;
    return geo.tiles * geo.tile_bytes;
}

int64_t q4_workspace_bytes(int32_t op, int32_t m, int32_t n, int32_t k)
{
    if (m < 1 || !valid_shape(n, k))
        return 0;
    if (op == Q4_OP_ATTENTION)   // m = ctx, n = query heads, k = head dim
        return (k % 32 == 0 && k <= 256) ? q4::attention_workspace_bytes(m, n, k) : 0;
    if (op == Q4_OP_LMHEAD) {
        q4::Geometry geo;
        if (!q4::layout_geometry(n, k, &geo))
            return 0;
        return q4::argmax_workspace_bytes(geo);
    }
    return 0;
}

int q4_layout_geometry(int32_t rows, int32_t k, int64_t *out)
{
    if (!out)
        return Q4_ERR_NULL;
    q4::Geometry geo;
    if (!valid_shape(rows, k) || !q4::layout_geometry(rows, k, &geo))
        return Q4_ERR_SHAPE;
    out[0] = geo.L;
    out[1] = geo.CG;
    out[2] = geo.P;
    out[3] = geo.TR;
    out[4] = geo.tiles;
    out[5] = geo.tile_bytes;
    return Q4_OK;
}

int q4_pack(const uint32_t *words, const uint16_t *scales, int32_t n, int32_t k, void *dst,
            int64_t dst_bytes, q4_weight *out, void *stream)
{
    return pack_common(words, scales, nullptr, nullptr, n, k, q4::PACK_ROWS, 0, dst, dst_bytes,
                       out, stream);
}

int q4_pack_rope(const uint32_t *words, const uint16_t *scales, int32_t n, int32_t k,
                 int32_t head_dim, void *dst, int64_t dst_bytes, q4_weight *out, void *stream)
{
    return pack_common(words, scales, nullptr, nullptr, n, k, q4::PACK_ROPE, head_dim, dst,
                       dst_bytes, out, stream);
}

int q4_pack_gate_up(const uint32_t *gw, const uint16_t *gs, const uint32_t *uw,
                    const uint16_t *us, int32_t n, int32_t k, void *dst, int64_t dst_bytes,
                    q4_weight *out, void *stream)
{
    return pack_common(gw, gs, uw, us, n, k, q4::PACK_GATE_UP, 0, dst, dst_bytes, out, stream);
}

// int3 packing; with (uw3, us) the gate/up interleave of (gw3, gs) and them
int pack3_common(const uint32_t *gw3, const uint16_t *gs, const uint32_t *uw3, const uint16_t *us,
                 int32_t n, int32_t k, void *dst, int64_t dst_bytes, q4_weight *out, void *stream)
{
    const bool gate_up = uw3 != nullptr || us != nullptr;
    if (!gw3 || !gs || !dst || !out || (gate_up && (!uw3 || !us)))
        return Q4_ERR_NULL;
    if (!valid_shape(n, k))
        return Q4_ERR_SHAPE;
    if (!aligned(gw3, 4) || !aligned(gs, 2) || !aligned(dst, 256) ||
        (gate_up && (!aligned(uw3, 4) || !aligned(us, 2))))
        return Q4_ERR_ALIGN;
    const int64_t rows = gate_up ? 2 * (int64_t)n : (int64_t)n;
    q4::Geometry geo;
    if (!q4::layout_geometry3(rows, k, &geo))
        return Q4_ERR_SHAPE;
    const int64_t need = geo.tiles * geo.tile_bytes;
    if (dst_bytes < need)
        return Q4_ERR_SIZE;
    const int64_t wbytes = (int64_t)n * (3 * (int64_t)k / 32) * 4, sbytes = (int64_t)n * (k / 32) * 2;
    if (overlap(dst, need, gw3, wbytes) || overlap(dst, need, gs, sbytes) ||
        (gate_up && (overlap(dst, need, uw3, wbytes) || overlap(dst, need, us, sbytes))))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    const int rc = hip_status(q4::launch_pack3(gw3, gs, gate_up ? uw3 : nullptr,
                                               gate_up ? us : nullptr, rows, k, geo, dst,
                                               static_cast<hipStream_t>(stream)));
    if (rc != Q4_OK)
        return rc;
    out->n = n;
    out->k = k;
    out->layout = gate_up ? Q4_LAYOUT_INT3_GATE_UP : Q4_LAYOUT_INT3;
    out->version = Q4_LAYOUT_VERSION;
    out->data = dst;
    out->bytes = need;
    out->head_dim = 0;
    out->reserved = 0;
    return Q4_OK;
}

int q4_pack_int3(const uint32_t *words3, const uint16_t *scales, int32_t n, int32_t k, void *dst,
                 int64_t dst_bytes, q4_weight *out, void *stream)
{
    return pack3_common(words3, scales, nullptr, nullptr, n, k, dst, dst_bytes, out, stream);
}

int q4_pack_int3_gate_up(const uint32_t *gw3, const uint16_t *gs, const uint32_t *uw3,
                         const uint16_t *us, int32_t n, int32_t k, void *dst, int64_t dst_bytes,
                         q4_weight *out, void *stream)
{
    if (!uw3 || !us)
        return Q4_ERR_NULL;
    return pack3_common(gw3, gs, uw3, us, n, k, dst, dst_bytes, out, stream);
}

int q4_unpack(const q4_weight *w, uint32_t *words, uint16_t *scales, void *stream)
{
    if (!w || !words || !scales)
        return Q4_ERR_NULL;
    if (w->layout != Q4_LAYOUT_ROWS && w->layout != Q4_LAYOUT_GATE_UP &&
        w->layout != Q4_LAYOUT_ROPE && w->layout != Q4_LAYOUT_INT3 &&
        w->layout != Q4_LAYOUT_INT3_GATE_UP)
        return Q4_ERR_LAYOUT;
    q4::Geometry geo;
    int64_t rows = 0;
    const int rc = check_weight(w, w->layout, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    const bool int3 = w->layout == Q4_LAYOUT_INT3 || w->layout == Q4_LAYOUT_INT3_GATE_UP;
    if (!aligned(words, int3 ? 4 : 16) || !aligned(scales, 2))
        return Q4_ERR_ALIGN;
    const int64_t wbytes = int3 ? rows * (3 * (int64_t)w->k / 32) * 4 : rows * w->k / 2;
    const int64_t sbytes = rows * (w->k / 32) * 2;
    if (overlap(words, wbytes, w->data, w->bytes) || overlap(scales, sbytes, w->data, w->bytes) ||
        overlap(words, wbytes, scales, sbytes))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    if (int3)
        return hip_status(q4::launch_unpack3(w->data, rows, w->k, geo, words, scales,
                                             static_cast<hipStream_t>(stream)));
    const q4::PackMode mode = w->layout == Q4_LAYOUT_GATE_UP ? q4::PACK_GATE_UP
                              : (w->layout == Q4_LAYOUT_ROPE ? q4::PACK_ROPE : q4::PACK_ROWS);
    return hip_status(q4::launch_unpack(w->data, rows, w->k, mode, w->head_dim, geo, words, scales,
                                        static_cast<hipStream_t>(stream)));
}

int q4_gemv(const q4_weight *w, const uint16_t *x, uint16_t *y, void *stream)
{
    q4::Geometry geo;
    int64_t rows = 0;
    if (!w || !x || !y)
        return Q4_ERR_NULL;
    // int4 rows or int3 rows
    const bool int3 = w->layout == Q4_LAYOUT_INT3;
    int rc = check_weight(w, int3 ? Q4_LAYOUT_INT3 : Q4_LAYOUT_ROWS, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    if (!aligned(x, 16) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    if (overlap(y, 2 * (int64_t)w->n, x, 2 * (int64_t)w->k) ||
        overlap(y, 2 * (int64_t)w->n, w->data, w->bytes))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    if (int3)
        return hip_status(q4::launch_gemv3(geo, q4::EPI_F16, w->data, x, y, rows, w->k, w->n,
                                           q4::ArgmaxScratch{nullptr, nullptr},
                                           static_cast<hipStream_t>(stream)));
    return hip_status(q4::launch_gemv_family(geo, q4::EPI_F16, w->data, x, y, rows, w->k, w->n,
                                             q4::ArgmaxScratch{nullptr, nullptr}, nullptr, nullptr,
                                             static_cast<hipStream_t>(stream)));
}

int q4_gemm_path(const q4_weight *w, const uint16_t *X, int32_t m, uint16_t *Y, int32_t path,
                 void *stream)
{
    q4::Geometry geo;
    int64_t rows = 0;
    if (!w || !X || !Y)
        return Q4_ERR_NULL;
    // int4 or int3 rows
    const bool int3 = w->layout == Q4_LAYOUT_INT3;
    int rc = check_weight(w, int3 ? Q4_LAYOUT_INT3 : Q4_LAYOUT_ROWS, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    if (m < 1)
        return Q4_ERR_SHAPE;
    if (path != Q4_GEMM_AUTO && path != Q4_GEMM_VALU && path != Q4_GEMM_MFMA)
        return Q4_ERR_SHAPE;
    if (!aligned(X, 16) || !aligned(Y, 2))
        return Q4_ERR_ALIGN;
    const int64_t ybytes = 2 * (int64_t)m * w->n, xbytes = 2 * (int64_t)m * w->k;
    if (overlap(Y, ybytes, X, xbytes) || overlap(Y, ybytes, w->data, w->bytes))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    // one activation row is the GEMV: its kernels stream W faster than the
    // GEMM's single-row VALU pass (they need y 4-byte aligned)
    if (path == Q4_GEMM_AUTO && m == 1 && aligned(Y, 4)) {
        const q4::ArgmaxScratch none{nullptr, nullptr};
        const hipStream_t st = static_cast<hipStream_t>(stream);
        if (int3)
            return hip_status(q4::launch_gemv3(geo, q4::EPI_F16, w->data, X, Y, rows, w->k, w->n, none, st));
        return hip_status(q4::launch_gemv_family(geo, q4::EPI_F16, w->data, X, Y, rows, w->k, w->n, none,
                                                 nullptr, nullptr, st));
    }
    return hip_status(q4::launch_gemm(geo, w->data, X, m, w->n, w->k, Y, path,
                                      static_cast<hipStream_t>(stream), int3));
}

int q4_gemm(const q4_weight *w, const uint16_t *X, int32_t m, uint16_t *Y, void *ws,
            int64_t ws_bytes, void *stream)
{
    (void)ws;
    (void)ws_bytes;
    return q4_gemm_path(w, X, m, Y, Q4_GEMM_AUTO, stream);
}

int q4_ffn_gate_up_silu(const q4_weight *w, const uint16_t *x, uint16_t *h, void *stream)
{
    q4::Geometry geo;
    int64_t rows = 0;
    if (!w || !x || !h)
        return Q4_ERR_NULL;
    // int4 or int3 gate/up pairs
    const bool int3 = w->layout == Q4_LAYOUT_INT3_GATE_UP;
    int rc = check_weight(w, int3 ? Q4_LAYOUT_INT3_GATE_UP : Q4_LAYOUT_GATE_UP, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    if (!aligned(x, 16) || !aligned(h, 2))
        return Q4_ERR_ALIGN;
    if (overlap(h, 2 * (int64_t)w->n, x, 2 * (int64_t)w->k) ||
        overlap(h, 2 * (int64_t)w->n, w->data, w->bytes))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    if (int3)
        return hip_status(q4::launch_gemv3(geo, q4::EPI_SILU, w->data, x, h, rows, w->k, w->n,
                                           q4::ArgmaxScratch{nullptr, nullptr},
                                           static_cast<hipStream_t>(stream)));
    return hip_status(q4::launch_gemv_family(geo, q4::EPI_SILU, w->data, x, h, rows, w->k, w->n,
                                             q4::ArgmaxScratch{nullptr, nullptr}, nullptr, nullptr,
                                             static_cast<hipStream_t>(stream)));
}

// The LM head; scratch = nullptr: the argmax candidates go to the
// library's static scratch array instead of the caller's workspace.
static int lmhead_common(const q4_weight *w, const uint16_t *x, float *logits, int32_t *argmax,
                         void *ws, int64_t ws_bytes, void *stream, bool static_scratch);

int q4_lmhead_f32(const q4_weight *w, const uint16_t *x, float *logits, int32_t *argmax,
                  void *ws, int64_t ws_bytes, void *stream)
{
    return lmhead_common(w, x, logits, argmax, ws, ws_bytes, stream, false);
}

static int lmhead_common(const q4_weight *w, const uint16_t *x, float *logits, int32_t *argmax,
                         void *ws, int64_t ws_bytes, void *stream, bool static_scratch)
{
    q4::Geometry geo;
    int64_t rows = 0;
    if (!w || !x || !logits)
        return Q4_ERR_NULL;
    // int4 or int3 rows
    const bool int3 = w->layout == Q4_LAYOUT_INT3;
    int rc = check_weight(w, int3 ? Q4_LAYOUT_INT3 : Q4_LAYOUT_ROWS, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    if (!aligned(x, 16) || !aligned(logits, 8) || (argmax && !aligned(argmax, 4)))
        return Q4_ERR_ALIGN;
    const int64_t lbytes = 4 * (int64_t)w->n;
    q4::ArgmaxScratch am{nullptr, nullptr};
    if (argmax) {
        const int64_t need = q4::argmax_workspace_bytes(geo);
        if (static_scratch) {
            // the static scratch replaces the workspace: a size check, and
            // its device address (taken once per device)
            if (need > kNoAllocScratchBytes)
                return Q4_ERR_WORKSPACE;
            ws = noalloc_scratch(&rc);
            if (!ws)
                return rc;
            ws_bytes = kNoAllocScratchBytes;
        }
        if (!ws || ws_bytes < need)
            return Q4_ERR_WORKSPACE;
        if (!aligned(ws, 256))
            return Q4_ERR_ALIGN;
        if (overlap(ws, need, x, 2 * (int64_t)w->k) || overlap(ws, need, w->data, w->bytes) ||
            overlap(ws, need, logits, lbytes) || overlap(ws, need, argmax, 4) ||
            overlap(argmax, 4, x, 2 * (int64_t)w->k) || overlap(argmax, 4, w->data, w->bytes) ||
            overlap(argmax, 4, logits, lbytes))
            return Q4_ERR_ALIAS;
        am.counters = static_cast<uint32_t *>(ws);
        am.partials = reinterpret_cast<unsigned long long *>(static_cast<uint8_t *>(ws) + q4::kArgmaxCounterBytes);
        am.result = argmax;
    }
    if (overlap(logits, lbytes, x, 2 * (int64_t)w->k) ||
        overlap(logits, lbytes, w->data, w->bytes))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    if (int3)
        return hip_status(q4::launch_gemv3(geo, q4::EPI_F32, w->data, x, logits, rows, w->k, w->n, am,
                                           static_cast<hipStream_t>(stream)));
    return hip_status(q4::launch_gemv_family(geo, q4::EPI_F32, w->data, x, logits, rows, w->k,
                                             w->n, am, nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

int q4_lmhead_f32_noalloc(const q4_weight *w, const uint16_t *x, float *logits, int32_t *argmax,
                          void *stream)
{
    return lmhead_common(w, x, logits, argmax, nullptr, 0, stream, true);
}

// Shared checks of the add + RMSNorm entry points; out is y (gemv) or h
// (ffn), n of them.
static int check_norm_args(const q4_weight *w, const uint16_t *x, const uint16_t *residual,
                           const uint16_t *gamma, float eps, const uint16_t *residual_out,
                           const void *out, int64_t out_bytes)
{
    if (!(eps >= 0.f) || !std::isfinite(eps))
        return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(gamma, 16) || (residual && !aligned(residual, 16)) ||
        (residual_out && !aligned(residual_out, 16)))
        return Q4_ERR_ALIGN;
    const int64_t kb = 2 * (int64_t)w->k;
    // outputs overlap no input and not each other
    const void *ins[4] = {x, residual, gamma, w->data};
    const int64_t inb[4] = {kb, kb, kb, w->bytes};
    for (int i = 0; i < 4; ++i) {
        if (!ins[i])
            continue;
        if (overlap(out, out_bytes, ins[i], inb[i]) ||
            (residual_out && overlap(residual_out, kb, ins[i], inb[i])))
            return Q4_ERR_ALIAS;
    }
    if (residual_out && overlap(residual_out, kb, out, out_bytes))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

int q4_add_rmsnorm_gemv(const q4_weight *w, const uint16_t *x, const uint16_t *residual,
                        const uint16_t *gamma, float eps, uint16_t *residual_out, uint16_t *y,
                        void *stream)
{
    q4::Geometry geo;
    int64_t rows = 0;
    if (!w || !x || !gamma || !y)
        return Q4_ERR_NULL;
    int rc = check_weight(w, Q4_LAYOUT_ROWS, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    if (!aligned(y, 4))
        return Q4_ERR_ALIGN;
    rc = check_norm_args(w, x, residual, gamma, eps, residual_out, y, 2 * (int64_t)w->n);
    if (rc != Q4_OK)
        return rc;
    const q4::NormArgs nm{residual, gamma, residual_out, eps};
    (void)hipGetLastError();
    return hip_status(q4::launch_gemv_family(geo, q4::EPI_F16, w->data, x, y, rows, w->k, w->n,
                                             q4::ArgmaxScratch{nullptr, nullptr}, &nm, nullptr,
                                             static_cast<hipStream_t>(stream)));
}

int q4_add_rmsnorm_ffn_gate_up_silu(const q4_weight *w, const uint16_t *x,
                                    const uint16_t *residual, const uint16_t *gamma, float eps,
                                    uint16_t *residual_out, uint16_t *h, void *stream)
{
    q4::Geometry geo;
    int64_t rows = 0;
    if (!w || !x || !gamma || !h)
        return Q4_ERR_NULL;
    int rc = check_weight(w, Q4_LAYOUT_GATE_UP, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    if (!aligned(h, 2))
        return Q4_ERR_ALIGN;
    rc = check_norm_args(w, x, residual, gamma, eps, residual_out, h, 2 * (int64_t)w->n);
    if (rc != Q4_OK)
        return rc;
    const q4::NormArgs nm{residual, gamma, residual_out, eps};
    (void)hipGetLastError();
    return hip_status(q4::launch_gemv_family(geo, q4::EPI_SILU, w->data, x, h, rows, w->k, w->n,
                                             q4::ArgmaxScratch{nullptr, nullptr}, &nm, nullptr,
                                             static_cast<hipStream_t>(stream)));
}

// The fused QKV step with an optional add + RMSNorm prologue (nm null: none).
static int qkv_rope_common(const q4_weight *w, const uint16_t *x, const q4::NormArgs *nm,
                           int32_t n_q_heads, int32_t pos, double rope_base, uint16_t *qkv,
                           uint16_t *kv_cache, const int32_t *page_table, int32_t n_pages,
                           void *stream)
{
    q4::Geometry geo;
    int64_t rows = 0;
    if (!w || !x || !qkv || (kv_cache && !page_table))
        return Q4_ERR_NULL;
    int rc = check_weight(w, Q4_LAYOUT_ROPE, &geo, &rows);
    if (rc != Q4_OK)
        return rc;
    const int64_t d = w->head_dim, heads = (int64_t)w->n / d;
    if (d > 512)   // the kernels keep d/2 RoPE twiddles in LDS
        return Q4_ERR_SHAPE;
    const int64_t nkv2 = heads - n_q_heads;
    if (n_q_heads < 0 || nkv2 < 0 || nkv2 % 2 != 0 || pos < 0 || !(rope_base > 0.0) ||
        !std::isfinite(rope_base) || (kv_cache && n_pages < 1))
        return Q4_ERR_SHAPE;
    const int64_t nkv = nkv2 / 2;
    if (!aligned(x, 16) || !aligned(qkv, 4) || (kv_cache && !aligned(kv_cache, 4)) ||
        (page_table && !aligned(page_table, 4)))
        return Q4_ERR_ALIGN;
    const int64_t kb = 2 * (int64_t)w->k, yb = 2 * (int64_t)w->n;
    const int64_t cb = (int64_t)n_pages * 2 * 16 * nkv * d * 2;
    const int64_t ptb = 4 * ((int64_t)pos / 16 + 1);
    if (overlap(qkv, yb, x, kb) || overlap(qkv, yb, w->data, w->bytes))
        return Q4_ERR_ALIAS;
    if (kv_cache && (overlap(kv_cache, cb, x, kb) || overlap(kv_cache, cb, w->data, w->bytes) ||
                     overlap(kv_cache, cb, qkv, yb) || overlap(kv_cache, cb, page_table, ptb)))
        return Q4_ERR_ALIAS;
    if (page_table && overlap(qkv, yb, page_table, ptb))
        return Q4_ERR_ALIAS;
    if (nm) {
        rc = check_norm_args(w, x, nm->r, nm->gamma, nm->eps, nm->h_out, qkv, yb);
        if (rc != Q4_OK)
            return rc;
        if (kv_cache && ((nm->r && overlap(kv_cache, cb, nm->r, kb)) ||
                         overlap(kv_cache, cb, nm->gamma, kb) ||
                         (nm->h_out && overlap(kv_cache, cb, nm->h_out, kb))))
            return Q4_ERR_ALIAS;
    }
    const q4::RopeArgs rp{(int32_t)d, n_q_heads, (int32_t)nkv, pos, rope_base, kv_cache,
                          page_table, n_pages};
    (void)hipGetLastError();
    return hip_status(q4::launch_gemv_family(geo, q4::EPI_ROPE, w->data, x, qkv, rows, w->k, w->n,
                                             q4::ArgmaxScratch{nullptr, nullptr}, nm, &rp,
                                             static_cast<hipStream_t>(stream)));
}

int q4_qkv_rope_append(const q4_weight *w, const uint16_t *x, int32_t n_q_heads, int32_t pos,
                       double rope_base, uint16_t *qkv, uint16_t *kv_cache,
                       const int32_t *page_table, int32_t n_pages, void *stream)
{
    return qkv_rope_common(w, x, nullptr, n_q_heads, pos, rope_base, qkv, kv_cache, page_table,
                           n_pages, stream);
}

int q4_add_rmsnorm_qkv_rope_append(const q4_weight *w, const uint16_t *x,
                                   const uint16_t *residual, const uint16_t *gamma, float eps,
                                   uint16_t *residual_out, int32_t n_q_heads, int32_t pos,
                                   double rope_base, uint16_t *qkv, uint16_t *kv_cache,
                                   const int32_t *page_table, int32_t n_pages, void *stream)
{
    if (!gamma)
        return Q4_ERR_NULL;
    const q4::NormArgs nm{residual, gamma, residual_out, eps};
    return qkv_rope_common(w, x, &nm, n_q_heads, pos, rope_base, qkv, kv_cache, page_table,
                           n_pages, stream);
}

int q4_attention_decode(const uint16_t *q, const uint16_t *kv_cache, const int32_t *page_table,
                        int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                        float scale, uint16_t *out, void *ws, int64_t ws_bytes, void *stream)
{
    if (!q || !kv_cache || !page_table || !out)
        return Q4_ERR_NULL;
    // one page of the cache (K and V halves) is addressed with 32-bit offsets
    if (ctx < 1 || n_pages < 1 || nq < 1 || nkv < 1 || nq % nkv != 0 || d < 32 || d > 256 ||
        d % 32 != 0 || !std::isfinite(scale) || (int64_t)nkv * 16 * d * 2 * 2 > INT32_MAX)
        return Q4_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(page_table, 4) || !aligned(out, 4) ||
        (ws && !aligned(ws, 16)))
        return Q4_ERR_ALIGN;
    const int64_t need = q4::attention_workspace_bytes(ctx, nq, d);
    if (need > 0 && (!ws || ws_bytes < need))
        return Q4_ERR_WORKSPACE;
    const int64_t qb = 2 * (int64_t)nq * d, cb = (int64_t)n_pages * 2 * 16 * nkv * d * 2;
    const int64_t tb = 4 * (((int64_t)ctx + 15) / 16);
    if (overlap(out, qb, q, qb) || overlap(out, qb, kv_cache, cb) || overlap(out, qb, page_table, tb))
        return Q4_ERR_ALIAS;
    if (need > 0 && (overlap(ws, need, q, qb) || overlap(ws, need, kv_cache, cb) ||
                     overlap(ws, need, page_table, tb) || overlap(ws, need, out, qb)))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    return hip_status(q4::launch_attention(q, kv_cache, page_table, n_pages, ctx, nq, nkv, d, scale,
                                           out, need > 0 ? ws : nullptr,
                                           static_cast<hipStream_t>(stream)));
}

int64_t q4_kv_int8_page_bytes(int32_t n_kv_heads, int32_t head_dim)
{
    if (n_kv_heads < 1 || head_dim < 32 || head_dim > 256 || head_dim % 32 != 0)
        return 0;
    const int64_t b = q4::kv_int8_page_bytes(n_kv_heads, head_dim);
    return b <= INT32_MAX ? b : 0;
}

int q4_kv_append_int8(const uint16_t *qkv, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      int32_t pos, void *cache8, const int32_t *page_table, int32_t n_pages,
                      void *stream)
{
    if (!qkv || !cache8 || !page_table)
        return Q4_ERR_NULL;
    const int64_t pb = q4_kv_int8_page_bytes(n_kv_heads, head_dim);
    if (pb == 0 || n_q_heads < 1 || pos < 0 || n_pages < 1)
        return Q4_ERR_SHAPE;
    if (!aligned(qkv, 2) || !aligned(cache8, 16) || !aligned(page_table, 4))
        return Q4_ERR_ALIGN;
    const int64_t qb = 2 * ((int64_t)n_q_heads + 2 * (int64_t)n_kv_heads) * head_dim;
    const int64_t cb = (int64_t)n_pages * pb, tb = 4 * ((int64_t)pos / 16 + 1);
    if (overlap(cache8, cb, qkv, qb) || overlap(cache8, cb, page_table, tb))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    return hip_status(q4::launch_kv_append_int8(qkv, n_q_heads, n_kv_heads, head_dim, pos,
                                                static_cast<uint8_t *>(cache8), page_table, n_pages,
                                                static_cast<hipStream_t>(stream)));
}

int q4_attention_decode_int8(const uint16_t *q, const void *cache8, const int32_t *page_table,
                             int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                             float scale, uint16_t *out, void *ws, int64_t ws_bytes, void *stream)
{
    if (!q || !cache8 || !page_table || !out)
        return Q4_ERR_NULL;
    const int64_t pb = q4_kv_int8_page_bytes(nkv, d);
    if (pb == 0 || ctx < 1 || n_pages < 1 || nq < 1 || nq % nkv != 0 || !std::isfinite(scale))
        return Q4_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(cache8, 16) || !aligned(page_table, 4) || !aligned(out, 4) ||
        (ws && !aligned(ws, 16)))
        return Q4_ERR_ALIGN;
    const int64_t need = q4::attention_workspace_bytes(ctx, nq, d);
    if (need > 0 && (!ws || ws_bytes < need))
        return Q4_ERR_WORKSPACE;
    const int64_t qb = 2 * (int64_t)nq * d, cb = (int64_t)n_pages * pb;
    const int64_t tb = 4 * (((int64_t)ctx + 15) / 16);
    if (overlap(out, qb, q, qb) || overlap(out, qb, cache8, cb) || overlap(out, qb, page_table, tb))
        return Q4_ERR_ALIAS;
    if (need > 0 && (overlap(ws, need, q, qb) || overlap(ws, need, cache8, cb) ||
                     overlap(ws, need, page_table, tb) || overlap(ws, need, out, qb)))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    return hip_status(q4::launch_attention_int8(q, static_cast<const uint8_t *>(cache8), page_table,
                                                n_pages, ctx, nq, nkv, d, scale, out,
                                                need > 0 ? ws : nullptr,
                                                static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ chain --

namespace {

struct ChainLayout {
    int64_t epochs, flags[q4::kChainMaxStages], tags[q4::kChainMaxStages], total;
};

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

// Workspace offsets: error word, per-block epochs, then the completion flags
// of every stage another waits `after`, and the tagged output of every stage
// another reads as `src`.
ChainLayout chain_layout(const q4_chain_stage *st, int32_t n)
{
    ChainLayout l{};
    int64_t off = 256;
    l.epochs = off;
    off += 4 * q4::kChainMaxBlocks;
    for (int i = 0; i < n; ++i) {
        bool waited = false, read = false;
        for (int j = i + 1; j < n; ++j) {
            waited |= st[j].after == i;
            read |= st[j].src == i;
        }
        l.flags[i] = -1;
        l.tags[i] = -1;
        if (waited) {
            l.flags[i] = off;
            off += 4 * q4::kChainMaxBlocks;
        }
        if (read) {
            l.tags[i] = off;
            off = align256(off + 4 * (int64_t)st[i].w->n);
        }
    }
    l.total = off;
    return l;
}

// Every check of q4_chain that does not involve the workspace; fills the
// kernel-side stage descriptors (pointers into the workspace left null).
int chain_check(const q4_chain_stage *st, int32_t n, q4::ChainArgs *a)
{
    if (!st)
        return Q4_ERR_NULL;
    if (n < 1 || n > q4::kChainMaxStages)
        return Q4_ERR_SHAPE;
    a->n_given = 0;
    for (int i = 0; i < n; ++i) {
        const q4_chain_stage &s = st[i];
        if (!s.w || !s.w->data || !s.y || (s.src < 0 && !s.x))
            return Q4_ERR_NULL;
        const bool gate_up = s.w->layout == Q4_LAYOUT_GATE_UP;
        if (!gate_up && s.w->layout != Q4_LAYOUT_ROWS)
            return Q4_ERR_LAYOUT;
        q4::Geometry geo;
        int64_t rows = 0;
        const int rc = check_weight(s.w, s.w->layout, &geo, &rows);
        if (rc != Q4_OK)
            return rc;
        const int g = q4::chain_geo_of(geo);
        if (g < 0)
            return Q4_ERR_SHAPE;   // k outside 1568 .. 8192 (or a geometry without a chain path)
        if (s.src >= i || s.after >= i || s.src < -1 || s.after < -1 || (s.src >= 0 && s.x))
            return Q4_ERR_SHAPE;
        if (s.src >= 0 && st[s.src].w && st[s.src].w->n != s.w->k)
            return Q4_ERR_SHAPE;
        if (s.gamma && (!(s.eps >= 0.f) || !std::isfinite(s.eps)))
            return Q4_ERR_SHAPE;
        if ((s.x && !aligned(s.x, 16)) || !aligned(s.y, gate_up ? 2 : 4) ||
            (s.gamma && !aligned(s.gamma, 16)) || (s.residual && !aligned(s.residual, 16)) ||
            (s.residual_out && !aligned(s.residual_out, 16)))
            return Q4_ERR_ALIGN;
        q4::ChainStageK &k = a->st[i];
        k = q4::ChainStageK{};
        k.wd = static_cast<const uint8_t *>(s.w->data);
        const bool dep = s.src >= 0;
        k.r = dep && s.gamma ? s.residual : nullptr;
        k.gamma = dep ? s.gamma : nullptr;
        k.h_out = dep && s.gamma ? s.residual_out : nullptr;
        k.y = s.y;
        if (!dep) {
            // a given x is staged once per launch; stages that read the same
            // vector with no prologue share it
            int g = -1;
            for (int j = 0; j < a->n_given && g < 0; ++j)
                if (!s.gamma && a->given[j].x == s.x && a->given[j].gamma == nullptr && a->given[j].k == s.w->k)
                    g = j;
            if (g < 0) {
                g = a->n_given++;
                const int off = g == 0 ? 0 : a->given[g - 1].off + a->given[g - 1].k / 8;
                if ((int64_t)off * 8 + s.w->k > q4::kChainGivenHalves)
                    return Q4_ERR_SHAPE;   // the given vectors exceed the staged-x area
                a->given[g] = q4::ChainGiven{s.x, s.gamma ? s.residual : nullptr, s.gamma,
                                             s.gamma ? s.residual_out : nullptr, s.eps, s.w->k, off};
            }
            k.xoff = a->given[g].off;
        }
        k.tiles = geo.tiles;
        k.rows = rows;
        k.n_out = s.w->n;
        k.k = s.w->k;
        k.geo = g;
        k.epi = gate_up ? q4::EPI_SILU : q4::EPI_F16;
        k.src = s.src;
        k.after = s.after;
        k.eps = s.eps;
    }
    // outputs overlap no input, no weight and no other output
    for (int i = 0; i < n; ++i) {
        const int64_t yb = 2 * (int64_t)st[i].w->n, kb = 2 * (int64_t)st[i].w->k;
        const void *outs[2] = {st[i].y, st[i].gamma ? st[i].residual_out : nullptr};
        const int64_t outb[2] = {yb, kb};
        for (int o = 0; o < 2; ++o) {
            if (!outs[o])
                continue;
            for (int j = 0; j < n; ++j) {
                const int64_t jk = 2 * (int64_t)st[j].w->k, jy = 2 * (int64_t)st[j].w->n;
                if (overlap(outs[o], outb[o], st[j].x, jk) || overlap(outs[o], outb[o], st[j].residual, jk) ||
                    overlap(outs[o], outb[o], st[j].gamma, jk) ||
                    overlap(outs[o], outb[o], st[j].w->data, st[j].w->bytes))
                    return Q4_ERR_ALIAS;
                if (j != i && (overlap(outs[o], outb[o], st[j].y, jy) ||
                               (st[j].gamma && overlap(outs[o], outb[o], st[j].residual_out, jk))))
                    return Q4_ERR_ALIAS;
            }
        }
        if (st[i].gamma && st[i].residual_out && overlap(st[i].y, yb, st[i].residual_out, kb))
            return Q4_ERR_ALIAS;
    }
    a->n = n;
    return Q4_OK;
}

}  // namespace

int64_t q4_chain_workspace_bytes(const q4_chain_stage *stages, int32_t n_stages)
{
    q4::ChainArgs a{};
    if (chain_check(stages, n_stages, &a) != Q4_OK)
        return 0;
    return chain_layout(stages, n_stages).total;
}

int q4_chain(const q4_chain_stage *stages, int32_t n_stages, void *ws, int64_t ws_bytes, void *stream)
{
    q4::ChainArgs a{};
    int rc = chain_check(stages, n_stages, &a);
    if (rc != Q4_OK)
        return rc;
    const ChainLayout l = chain_layout(stages, n_stages);
    if (!ws || ws_bytes < l.total)
        return Q4_ERR_WORKSPACE;
    if (!aligned(ws, 256))
        return Q4_ERR_ALIGN;
    for (int i = 0; i < n_stages; ++i) {
        const q4_chain_stage &s = stages[i];
        const int64_t kb = 2 * (int64_t)s.w->k;
        if (overlap(ws, l.total, s.x, kb) || overlap(ws, l.total, s.residual, kb) ||
            overlap(ws, l.total, s.gamma, kb) || overlap(ws, l.total, s.w->data, s.w->bytes) ||
            overlap(ws, l.total, s.y, 2 * (int64_t)s.w->n) ||
            (s.gamma && overlap(ws, l.total, s.residual_out, kb)))
            return Q4_ERR_ALIAS;
    }
    const int blocks = q4::device_cus();
    if (blocks > q4::kChainMaxBlocks)
        return Q4_ERR_SHAPE;
    uint8_t *base = static_cast<uint8_t *>(ws);
    a.error = reinterpret_cast<uint32_t *>(base);
    a.epochs = reinterpret_cast<uint32_t *>(base + l.epochs);
    for (int i = 0; i < n_stages; ++i) {
        a.st[i].flags = l.flags[i] >= 0 ? reinterpret_cast<uint32_t *>(base + l.flags[i]) : nullptr;
        a.st[i].tag = l.tags[i] >= 0 ? reinterpret_cast<uint32_t *>(base + l.tags[i]) : nullptr;
    }
    a.wait_ticks = 200000;   // 2 ms of the 100 MHz device clock
    (void)hipGetLastError();
    return hip_status(q4::launch_chain(a, blocks, static_cast<hipStream_t>(stream)));
}

int q4_read_probe(const void *src, int64_t bytes, uint32_t *sink, int64_t sink_bytes, void *stream)
{
    if (!src || !sink)
        return Q4_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0)
        return Q4_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(sink, 4))
        return Q4_ERR_ALIGN;
    const int cus = q4::device_cus();
    if (sink_bytes < 4 * q4::read_probe_blocks(bytes, cus))
        return Q4_ERR_SIZE;
    if (overlap(sink, sink_bytes, src, bytes))
        return Q4_ERR_ALIAS;
    (void)hipGetLastError();
    return hip_status(q4::launch_read_probe(src, bytes, sink, cus, static_cast<hipStream_t>(stream)));
}

const char *q4_strerror(int code)
{
    switch (code) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "invalid shape (n < 1, k < 32, k % 32 != 0, m < 1 or too large)";
    case Q4_ERR_ALIGN: return "a pointer is not aligned as documented";
    case Q4_ERR_LAYOUT: return "weight layout or layout version does not suit this call";
    case Q4_ERR_WORKSPACE: return "workspace missing or smaller than q4_workspace_bytes";
    case Q4_ERR_ALIAS: return "an output range overlaps an input range";
    case Q4_ERR_HIP: return "the HIP runtime refused the launch (see q4_last_hip_error)";
    case Q4_ERR_SIZE: return "a destination buffer is smaller than required";
    }
    return "unknown q4 error code";
}

int q4_last_hip_error(void) { return g_last_hip_error; }

#ifndef Q4_SOURCE_HASH
#define Q4_SOURCE_HASH "unstamped"
#endif
const char *q4_source_hash(void) { return Q4_SOURCE_HASH; }

}  // extern "C"
