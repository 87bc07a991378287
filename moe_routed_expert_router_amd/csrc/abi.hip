// C ABI entry points: argument and geometry validation on the host, then the
// kernel launches on the caller's stream.  Nothing is enqueued after a failed
// check (the 96 GB RTX PRO 6000 write-up, "Five layers made the difference",
// audits its host pages and pointers and fails startup when the geometry is
// wrong; the inference-engineering write-up's flag table records a setting
// whose pattern matched no parameter at all without any error — every
// malformed input here is an explicit status instead).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "kernels.hpp"

namespace {

thread_local char g_err[512];

moe_status fail(moe_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

moe_status ok() {
    g_err[0] = 0;
    return MOE_OK;
}

moe_status check_shape(const moe_shape *s) {
    if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    if (s->hidden <= 0 || s->inter <= 0 || s->n_experts <= 0 || s->top_k <= 0)
        return fail(MOE_ERR_INVALID_ARG, "shape fields must be positive (H=%d I=%d E=%d k=%d)", s->hidden,
                    s->inter, s->n_experts, s->top_k);
    if (s->hidden % 128 || s->inter % 128)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H and I must be multiples of 128 (H=%d I=%d)", s->hidden, s->inter);
    if (s->hidden > (1 << 16) || s->inter > (1 << 16))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H and I must be <= 65536");
    if (s->n_experts > moe::kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", s->n_experts, moe::kMaxExperts);
    if (s->top_k > moe::kMaxTopK || s->top_k > s->n_experts)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "k=%d must be <= min(E, %d)", s->top_k, moe::kMaxTopK);
    return MOE_OK;
}

moe_status check_tokens(int32_t T) {
    if (T < 0 || T > (1 << 20)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "n_tokens=%d outside [0, 2^20]", T);
    return MOE_OK;
}

// A pointer the GPU will dereference: not NULL, aligned, known to the HIP
// runtime as device memory or device-mapped host memory, and (where the runtime
// reports the allocation's range) with `bytes` bytes inside that allocation.
moe_status check_ptr(const void *p, size_t bytes, size_t align, const char *name) {
    if (!p) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    if ((uintptr_t)p % align) return fail(MOE_ERR_MISALIGNED, "%s is not %zu-byte aligned", name, align);
    hipPointerAttribute_t at;
    hipError_t e = hipPointerGetAttributes(&at, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_ERR_NOT_DEVICE_ACCESSIBLE, "%s (%p) is not memory known to HIP (%s)", name, p,
                    hipGetErrorString(e));
    }
    if (at.type == hipMemoryTypeUnregistered)
        return fail(MOE_ERR_NOT_DEVICE_ACCESSIBLE, "%s (%p) is unregistered host memory", name, p);
    if (at.type == hipMemoryTypeHost && at.devicePointer == nullptr)
        return fail(MOE_ERR_NOT_DEVICE_ACCESSIBLE, "%s (%p) is host memory not mapped for the device", name, p);
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    e = hipMemGetAddressRange(&base, &size, const_cast<void *>(p));
    if (e == hipSuccess && base != nullptr && size > 0) {
        const uintptr_t b = (uintptr_t)base, q = (uintptr_t)p;
        if (q < b || q + bytes > b + size)
            return fail(MOE_ERR_INVALID_ARG, "%s: %zu bytes at %p overrun its allocation (%zu bytes at %p)", name,
                        bytes, p, size, base);
    } else {
        (void)hipGetLastError();
    }
    return MOE_OK;
}

#define TRY(expr)                                   \
    do {                                            \
        moe_status _st = (expr);                    \
        if (_st != MOE_OK) return _st;              \
    } while (0)

moe_status check_ws(const moe_shape *s, int32_t T, void *ws, size_t ws_bytes) {
    const size_t need = moe::WsLayout::make(s->hidden, s->inter, s->n_experts, s->top_k, T).total;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    return check_ptr(ws, need, 256, "ws");
}

moe_status check_residency(const moe_shape *s, const moe_residency *r) {
    if (!r) return fail(MOE_ERR_INVALID_ARG, "residency is NULL");
    if (r->n_hot < 0 || r->n_cold < 0 || r->n_hot + r->n_cold != s->n_experts)
        return fail(MOE_ERR_BAD_RESIDENCY, "n_hot=%d + n_cold=%d must equal E=%d", r->n_hot, r->n_cold,
                    s->n_experts);
    const size_t B = moe::BlobLayout::make(s->hidden, s->inter).bytes;
    TRY(check_ptr(r->slot, (size_t)s->n_experts * 4, 4, "residency.slot"));
    if (r->n_hot > 0) TRY(check_ptr(r->hot_base, (size_t)r->n_hot * B, 16, "residency.hot_base"));
    if (r->n_cold > 0) {
        TRY(check_ptr(r->host_cold, (size_t)r->n_cold * B, 16, "residency.host_cold"));
        TRY(check_ptr(r->scratch, (size_t)r->n_cold * B, 16, "residency.scratch"));
    }
    return MOE_OK;
}

// Direct read: the cold experts are read in place from pinned host memory
// (the caller passed the host pool as the scratch), so nothing is gathered.
bool direct_read(const moe_residency *r) { return r->n_cold > 0 && r->scratch == r->host_cold; }

moe_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        (void)hipGetLastError();   // reported here: do not leave it for the caller's next HIP call
        return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    }
    return MOE_OK;
}

moe::GroupArgs group_args(const moe_shape *s, int32_t T, const int32_t *ids, const moe_residency *r) {
    moe::GroupArgs g;
    g.ids = ids;
    g.T = T;
    g.k = s->top_k;
    g.E = s->n_experts;
    g.slot = r->slot;
    g.n_hot = r->n_hot;
    g.n_cold = r->n_cold;
    g.hot_base = r->hot_base;
    g.scratch = r->scratch;
    g.blob_bytes = moe::BlobLayout::make(s->hidden, s->inter).bytes;
    return g;
}

moe::FfnArgs ffn_args(const moe_shape *s, int32_t T, const uint16_t *x, const int32_t *ids, const float *w,
                      int32_t out_dtype, void *out) {
    moe::FfnArgs a;
    a.x = x;
    a.ids = ids;
    a.w = w;
    a.T = T;
    a.H = s->hidden;
    a.I = s->inter;
    a.E = s->n_experts;
    a.k = s->top_k;
    a.out_bf16 = out_dtype == MOE_OUT_BF16;
    a.out = out;
    return a;
}

moe_status enqueue_ffn(const moe_shape *s, int32_t T, const uint16_t *x, const int32_t *ids, const float *w,
                       int32_t out_dtype, void *out, char *ws, const moe::WsLayout &L, hipStream_t st) {
    return hip_status(moe::launch_ffn(ffn_args(s, T, x, ids, w, out_dtype, out), ws, L, st), "ffn launch");
}

// Per-device side stream on which moe_layer_forward runs the cold gather while
// the hot experts' FFN runs on the caller's stream.  Created on first use with
// the default priority; the fork and join are event waits, so the pattern is
// also valid under stream capture.  The mutex keeps one call's record/wait
// pairs together when several host threads drive the same device.
struct SideStream {
    std::mutex mu;
    hipStream_t st = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];

moe_status side_stream(std::unique_lock<std::mutex> &lock, SideStream **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return fail(MOE_ERR_HIP, "no usable current device for the gather stream");
    }
    SideStream &s = g_side[dev];
    lock = std::unique_lock<std::mutex>(s.mu);
    if (s.st == nullptr) {
        hipStream_t st = nullptr;
        hipEvent_t a = nullptr, b = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
            const hipError_t e = hipGetLastError();
            if (b) (void)hipEventDestroy(b);
            if (a) (void)hipEventDestroy(a);
            if (st) (void)hipStreamDestroy(st);
            return fail(MOE_ERR_HIP, "gather stream setup: %s", hipGetErrorString(e));
        }
        s.st = st;
        s.fork = a;
        s.join = b;
    }
    *out = &s;
    return MOE_OK;
}

// Workspace of moe_layer_forward_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  Its host-
// side name is not a device address: the kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on that entry point's first call there.
static __device__ __align__(256) uint8_t noalloc_scratch[MOE_NOALLOC_WS_BYTES];

struct NoallocWs {
    std::once_flag once;
    hipError_t err = hipSuccess;
    void *ptr = nullptr;
};
NoallocWs g_noalloc[kMaxDevices];

moe_status noalloc_ws(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return fail(MOE_ERR_HIP, "no usable current device for the static workspace");
    }
    NoallocWs &w = g_noalloc[dev];
    std::call_once(w.once, [&w] {
        void *p = nullptr;
        w.err = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
        w.ptr = w.err == hipSuccess ? p : nullptr;
        if (w.err != hipSuccess) (void)hipGetLastError();
    });
    if (w.err != hipSuccess || w.ptr == nullptr)
        return fail(MOE_ERR_HIP, "static workspace address on device %d: %s", dev, hipGetErrorString(w.err));
    *out = w.ptr;
    return MOE_OK;
}

moe_status check_out(const moe_shape *s, int32_t T, int32_t out_dtype, void *out) {
    if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16)
        return fail(MOE_ERR_INVALID_ARG, "out_dtype %d unknown", out_dtype);
    return check_ptr(out, (size_t)T * s->hidden * (out_dtype == MOE_OUT_F32 ? 4 : 2), 16, "out");
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status st) {
    switch (st) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
        case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
        case MOE_ERR_NOT_DEVICE_ACCESSIBLE: return "MOE_ERR_NOT_DEVICE_ACCESSIBLE";
        case MOE_ERR_BAD_RESIDENCY: return "MOE_ERR_BAD_RESIDENCY";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char *moe_last_error(void) { return g_err; }

moe_status moe_shape_check(const moe_shape *s) {
    TRY(check_shape(s));
    return ok();
}

size_t moe_expert_bytes(const moe_shape *s) {
    if (check_shape(s) != MOE_OK) return 0;
    return moe::BlobLayout::make(s->hidden, s->inter).bytes;
}

size_t moe_workspace_bytes(const moe_shape *s, int32_t n_tokens) {
    if (check_shape(s) != MOE_OK || check_tokens(n_tokens) != MOE_OK) return 0;
    return moe::WsLayout::make(s->hidden, s->inter, s->n_experts, s->top_k, n_tokens).total;
}

moe_status moe_residency_check(const moe_shape *s, const int32_t *slot_host, int32_t n_hot, int32_t n_cold) {
    TRY(check_shape(s));
    if (!slot_host) return fail(MOE_ERR_INVALID_ARG, "slot_host is NULL");
    const int E = s->n_experts;
    if (n_hot < 0 || n_cold < 0 || n_hot + n_cold != E)
        return fail(MOE_ERR_BAD_RESIDENCY, "n_hot=%d + n_cold=%d must equal E=%d", n_hot, n_cold, E);
    static thread_local unsigned char seen[2 * moe::kMaxExperts];
    memset(seen, 0, sizeof(seen));
    for (int e = 0; e < E; ++e) {
        const int32_t v = slot_host[e];
        if (v >= 0) {
            if (v >= n_hot || seen[v]) return fail(MOE_ERR_BAD_RESIDENCY, "expert %d: hot index %d invalid or repeated", e, v);
            seen[v] = 1;
        } else {
            const int64_t c = -(int64_t)v - 1;
            if (c >= n_cold || seen[moe::kMaxExperts + c])
                return fail(MOE_ERR_BAD_RESIDENCY, "expert %d: cold slot %lld invalid or repeated", e, (long long)c);
            seen[moe::kMaxExperts + c] = 1;
        }
    }
    return ok();
}

moe_status moe_host_alloc(size_t bytes, int32_t flags, void **host_ptr, void **device_ptr) {
    if (!host_ptr || !device_ptr || bytes == 0) return fail(MOE_ERR_INVALID_ARG, "bad moe_host_alloc arguments");
    *host_ptr = nullptr;
    *device_ptr = nullptr;
    const unsigned f = hipHostMallocMapped | hipHostMallocPortable |
                       ((flags & 1) ? hipHostMallocCoherent : hipHostMallocNonCoherent);
    void *h = nullptr;
    hipError_t e = hipHostMalloc(&h, bytes, f);
    if (e != hipSuccess) return hip_status(e, "hipHostMalloc");
    void *d = nullptr;
    e = hipHostGetDevicePointer(&d, h, 0);
    if (e != hipSuccess) {
        (void)hipHostFree(h);
        return hip_status(e, "hipHostGetDevicePointer");
    }
    *host_ptr = h;
    *device_ptr = d;
    return ok();
}

moe_status moe_host_free(void *host_ptr) {
    if (!host_ptr) return fail(MOE_ERR_INVALID_ARG, "host_ptr is NULL");
    TRY(hip_status(hipHostFree(host_ptr), "hipHostFree"));
    return ok();
}

moe_status moe_route(const moe_shape *s, int32_t T, const uint16_t *x, const float *w_router, const float *bias,
                     int32_t renormalize, int32_t *topk_ids, float *topk_w, float *logits_out, void *ws,
                     size_t ws_bytes, void *stream) {
    TRY(check_shape(s));
    TRY(check_tokens(T));
    if (T == 0) return ok();
    const int H = s->hidden, E = s->n_experts, k = s->top_k;
    TRY(check_ptr(x, (size_t)T * H * 2, 16, "x"));
    TRY(check_ptr(w_router, (size_t)E * H * 4, 16, "w_router"));
    if (bias) TRY(check_ptr(bias, (size_t)E * 4, 4, "bias"));
    TRY(check_ptr(topk_ids, (size_t)T * k * 4, 4, "topk_ids"));
    TRY(check_ptr(topk_w, (size_t)T * k * 4, 4, "topk_w"));
    if (logits_out) TRY(check_ptr(logits_out, (size_t)T * E * 4, 4, "logits_out"));
    TRY(check_ws(s, T, ws, ws_bytes));
    const moe::WsLayout L = moe::WsLayout::make(H, s->inter, E, k, T);
    float *z = logits_out ? logits_out : reinterpret_cast<float *>(static_cast<char *>(ws) + L.logits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    TRY(hip_status(moe::launch_route_logits(x, w_router, bias, T, H, E, z, st), "router logits launch"));
    TRY(hip_status(moe::launch_topk(z, T, E, k, renormalize != 0, topk_ids, topk_w, st), "top-k launch"));
    return ok();
}

moe_status moe_pick_set(const moe_shape *s, int32_t T, const int32_t *topk_ids, const int32_t *slot, int32_t n_hot,
                        int32_t n_cold, int32_t *counts_out, int32_t *cold_out, void *ws, size_t ws_bytes,
                        void *stream) {
    TRY(check_shape(s));
    TRY(check_tokens(T));
    const int E = s->n_experts, k = s->top_k;
    if (n_hot < 0 || n_cold < 0 || n_hot + n_cold != E)
        return fail(MOE_ERR_BAD_RESIDENCY, "n_hot=%d + n_cold=%d must equal E=%d", n_hot, n_cold, E);
    if (T > 0) TRY(check_ptr(topk_ids, (size_t)T * k * 4, 4, "topk_ids"));
    TRY(check_ptr(slot, (size_t)E * 4, 4, "slot"));
    TRY(check_ptr(counts_out, (size_t)E * 4, 4, "counts_out"));
    TRY(check_ptr(cold_out, (size_t)(E + 1) * 4, 4, "cold_out"));
    TRY(check_ws(s, T, ws, ws_bytes));
    const moe::WsLayout L = moe::WsLayout::make(s->hidden, s->inter, E, k, T);
    char *w = static_cast<char *>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    moe_residency r;
    r.slot = slot;
    r.n_hot = n_hot;
    r.n_cold = n_cold;
    // only the index ranges matter here: the address table is not used
    r.hot_base = reinterpret_cast<const uint8_t *>(w);
    r.scratch = reinterpret_cast<uint8_t *>(w);
    r.host_cold = nullptr;
    TRY(hip_status(moe::launch_group(group_args(s, T, topk_ids, &r), w, L, st), "pick-set launch"));
    TRY(hip_status(moe::launch_pick_set_out(w, L, E, counts_out, cold_out, st), "pick-set output launch"));
    return ok();
}

moe_status moe_gather_cold(const moe_shape *s, int32_t T, const int32_t *topk_ids, const moe_residency *r, void *ws,
                           size_t ws_bytes, void *stream) {
    TRY(check_shape(s));
    TRY(check_tokens(T));
    TRY(check_residency(s, r));
    if (T == 0 || r->n_cold == 0 || direct_read(r)) return ok();
    TRY(check_ptr(topk_ids, (size_t)T * s->top_k * 4, 4, "topk_ids"));
    TRY(check_ws(s, T, ws, ws_bytes));
    const moe::WsLayout L = moe::WsLayout::make(s->hidden, s->inter, s->n_experts, s->top_k, T);
    char *w = static_cast<char *>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const moe::GroupArgs g = group_args(s, T, topk_ids, r);
    TRY(hip_status(moe::launch_group(g, w, L, st), "pick-set launch"));
    TRY(hip_status(moe::launch_gather(r->host_cold, r->scratch, g.blob_bytes, r->slot, w, L, st), "gather launch"));
    return ok();
}

moe_status moe_expert_ffn(const moe_shape *s, int32_t T, const uint16_t *x, const int32_t *topk_ids,
                          const float *topk_w, const moe_residency *r, int32_t out_dtype, void *out, void *ws,
                          size_t ws_bytes, void *stream) {
    TRY(check_shape(s));
    TRY(check_tokens(T));
    TRY(check_residency(s, r));
    if (T == 0) return ok();
    const int k = s->top_k;
    TRY(check_ptr(x, (size_t)T * s->hidden * 2, 16, "x"));
    TRY(check_ptr(topk_ids, (size_t)T * k * 4, 4, "topk_ids"));
    TRY(check_ptr(topk_w, (size_t)T * k * 4, 4, "topk_w"));
    TRY(check_out(s, T, out_dtype, out));
    TRY(check_ws(s, T, ws, ws_bytes));
    const moe::WsLayout L = moe::WsLayout::make(s->hidden, s->inter, s->n_experts, k, T);
    char *w = static_cast<char *>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    TRY(hip_status(moe::launch_group(group_args(s, T, topk_ids, r), w, L, st), "pick-set launch"));
    TRY(enqueue_ffn(s, T, x, topk_ids, topk_w, out_dtype, out, w, L, st));
    return ok();
}

// (token, pick) pairs up to which a decode layer with cold experts runs the
// gather in order with the FFN rather than beside it on a second stream.
constexpr int kGatherOverlapMinPairs = 24;

// The layer's launch sequence on `stream`, after the arguments were checked.
// side_ok: the decode path with many cold picks may overlap the gather on
// the library's side stream; otherwise everything runs in order on `stream`
// (the same kernels and results).
static moe_status layer_forward_enqueue(const moe_shape *s, int32_t T, const uint16_t *x, const float *w_router,
                                        const float *bias, int32_t renormalize, const moe_residency *r,
                                        int32_t *topk_ids, float *topk_w, int32_t out_dtype, void *out, void *ws,
                                        void *stream, bool side_ok) {
    const int H = s->hidden, E = s->n_experts, k = s->top_k;
    const moe::WsLayout L = moe::WsLayout::make(H, s->inter, E, k, T);
    char *w = static_cast<char *>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    float *z = reinterpret_cast<float *>(w + L.logits);
    const moe::GroupArgs g = group_args(s, T, topk_ids, r);
    TRY(hip_status(moe::launch_route_logits(x, w_router, bias, T, H, E, z, st), "router logits launch"));
    const bool direct = direct_read(r);
    if (T <= moe::kSmallRouteTokens && (r->n_cold == 0 || direct) && moe::ffn_select_fusable(T, k, E, H, s->inter)) {
        // no cold expert to gather: the gate/up kernel selects and groups by itself
        const moe::FfnArgs a = ffn_args(s, T, x, topk_ids, topk_w, out_dtype, out);
        TRY(hip_status(moe::launch_ffn_select(a, z, renormalize != 0, topk_ids, topk_w, g, w, L, st),
                       "select + ffn launch"));
        return ok();
    }
    if (T <= moe::kSmallRouteTokens && r->n_cold > 0 && !direct && moe::ffn_select_fusable(T, k, E, H, s->inter)) {
        // one token with cold experts, all on the caller's stream: the hot
        // experts' gate/up (its blocks select and publish the pick set), the
        // gather of the published cold list, then the cold experts' gate/up
        // and the down projection with the combine.  Measured against running
        // a self-selecting gather beside the hot gate/up on a second stream:
        // that overlap slows the gate/up by more than it hides (per layer
        // with nothing cold 50.7 against 37.7 us; the 40-layer one-stream
        // step 3.00 against 2.48 ms)
        const moe::FfnArgs a = ffn_args(s, T, x, topk_ids, topk_w, out_dtype, out);
        const int P = T * k;
        TRY(hip_status(moe::launch_ffn_select_hot(a, z, renormalize != 0, topk_ids, topk_w, g, w, L, st),
                       "hot ffn launch"));
        TRY(hip_status(moe::launch_gather(r->host_cold, r->scratch, g.blob_bytes, r->slot, w, L, st),
                       "gather launch"));
        TRY(hip_status(moe::launch_ffn_part(a, moe::kPartCold, r->n_cold < P ? r->n_cold : P, w, L, st),
                       "cold ffn launch"));
        return ok();
    }
    if (T <= moe::kSmallRouteTokens && r->n_cold > 0 && !direct && moe::ffn_block_path(T, H, s->inter) &&
        (T * k <= kGatherOverlapMinPairs || !side_ok)) {
        // a few tokens with cold experts, in order on the caller's stream:
        // select and group, the hot experts' FFN, the gather of the published
        // cold list, the cold experts' FFN and the combine.  Measured per
        // layer against the side-stream overlap below: 59 against 75 us at 2
        // tokens, 83 against 98 at 4; the overlap wins from 8 tokens on (173
        // against 189)
        const moe::FfnArgs a = ffn_args(s, T, x, topk_ids, topk_w, out_dtype, out);
        const int P = T * k;
        TRY(hip_status(moe::launch_select_group_small(z, T, k, renormalize != 0, topk_ids, topk_w, g, w, L, st),
                       "select-and-group launch"));
        TRY(hip_status(moe::launch_ffn_part(a, moe::kPartHot, E < P ? E : P, w, L, st), "hot ffn launch"));
        TRY(hip_status(moe::launch_gather(r->host_cold, r->scratch, g.blob_bytes, r->slot, w, L, st),
                       "gather launch"));
        TRY(hip_status(moe::launch_ffn_part(a, moe::kPartCold, r->n_cold < P ? r->n_cold : P, w, L, st),
                       "cold ffn launch"));
        return ok();
    }
    if (T <= moe::kSmallRouteTokens && r->n_cold > 0 && !direct && moe::ffn_block_path(T, H, s->inter)) {
        // decode with cold experts, more tokens: the gather, forked right
        // after the router, takes the top-k from the logits itself on the
        // side stream, so it waits for no grouping; one select-and-group
        // launch and the hot experts' FFN run meanwhile on the caller's
        // stream; the cold experts' FFN and the combine follow the join
        const moe::FfnArgs a = ffn_args(s, T, x, topk_ids, topk_w, out_dtype, out);
        const int P = T * k;
        std::unique_lock<std::mutex> lock;
        SideStream *side = nullptr;
        TRY(side_stream(lock, &side));
        TRY(hip_status(hipEventRecord(side->fork, st), "gather fork"));
        TRY(hip_status(hipStreamWaitEvent(side->st, side->fork, 0), "gather fork"));
        TRY(hip_status(moe::launch_gather_sel(z, T, E, k, r->slot, r->n_cold, r->host_cold, r->scratch, g.blob_bytes,
                                              side->st),
                       "gather launch"));
        TRY(hip_status(hipEventRecord(side->join, side->st), "gather join"));
        TRY(hip_status(moe::launch_select_group_small(z, T, k, renormalize != 0, topk_ids, topk_w, g, w, L, st),
                       "select-and-group launch"));
        TRY(hip_status(moe::launch_ffn_part(a, moe::kPartHot, E < P ? E : P, w, L, st), "hot ffn launch"));
        TRY(hip_status(hipStreamWaitEvent(st, side->join, 0), "gather join"));
        lock.unlock();
        TRY(hip_status(moe::launch_ffn_part(a, moe::kPartCold, r->n_cold < P ? r->n_cold : P, w, L, st),
                       "cold ffn launch"));
        return ok();
    }
    if (T <= moe::kSmallRouteTokens) {
        TRY(hip_status(moe::launch_select_group_small(z, T, k, renormalize != 0, topk_ids, topk_w, g, w, L, st),
                       "select-and-group launch"));
    } else {
        TRY(hip_status(moe::launch_topk(z, T, E, k, renormalize != 0, topk_ids, topk_w, st), "top-k launch"));
        TRY(hip_status(moe::launch_group(g, w, L, st), "pick-set launch"));
    }
    if (r->n_cold > 0 && !direct)
        TRY(hip_status(moe::launch_gather(r->host_cold, r->scratch, g.blob_bytes, r->slot, w, L, st),
                       "gather launch"));
    TRY(enqueue_ffn(s, T, x, topk_ids, topk_w, out_dtype, out, w, L, st));
    return ok();
}

static moe_status check_layer_args(const moe_shape *s, int32_t T, const uint16_t *x, const float *w_router,
                                   const float *bias, const moe_residency *r, int32_t *topk_ids, float *topk_w,
                                   int32_t out_dtype, void *out) {
    TRY(check_shape(s));
    TRY(check_tokens(T));
    TRY(check_residency(s, r));
    if (T == 0) return MOE_OK;
    const int H = s->hidden, E = s->n_experts, k = s->top_k;
    TRY(check_ptr(x, (size_t)T * H * 2, 16, "x"));
    TRY(check_ptr(w_router, (size_t)E * H * 4, 16, "w_router"));
    if (bias) TRY(check_ptr(bias, (size_t)E * 4, 4, "bias"));
    TRY(check_ptr(topk_ids, (size_t)T * k * 4, 4, "topk_ids"));
    TRY(check_ptr(topk_w, (size_t)T * k * 4, 4, "topk_w"));
    TRY(check_out(s, T, out_dtype, out));
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_shape *s, int32_t T, const uint16_t *x, const float *w_router,
                             const float *bias, int32_t renormalize, const moe_residency *r, int32_t *topk_ids,
                             float *topk_w, int32_t out_dtype, void *out, void *ws, size_t ws_bytes,
                             void *stream) {
    TRY(check_layer_args(s, T, x, w_router, bias, r, topk_ids, topk_w, out_dtype, out));
    if (T == 0) return ok();
    TRY(check_ws(s, T, ws, ws_bytes));
    TRY(layer_forward_enqueue(s, T, x, w_router, bias, renormalize, r, topk_ids, topk_w, out_dtype, out, ws, stream,
                              true));
    return ok();
}

moe_status moe_layer_forward_noalloc(const moe_shape *s, int32_t T, const uint16_t *x, const float *w_router,
                                     const float *bias, int32_t renormalize, const moe_residency *r,
                                     int32_t *topk_ids, float *topk_w, int32_t out_dtype, void *out, void *stream) {
    TRY(check_layer_args(s, T, x, w_router, bias, r, topk_ids, topk_w, out_dtype, out));
    if (T == 0) return ok();
    const size_t need = moe::WsLayout::make(s->hidden, s->inter, s->n_experts, s->top_k, T).total;
    if (need > (size_t)MOE_NOALLOC_WS_BYTES)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                    "%d tokens need a %zu-byte workspace; the static one holds %zu (use moe_layer_forward)", T,
                    need, (size_t)MOE_NOALLOC_WS_BYTES);
    void *ws = nullptr;
    TRY(noalloc_ws(&ws));
    TRY(layer_forward_enqueue(s, T, x, w_router, bias, renormalize, r, topk_ids, topk_w, out_dtype, out, ws, stream,
                              false));
    return ok();
}

moe_status moe_count_picks(const moe_shape *s, int32_t T, const int32_t *topk_ids, int32_t *counts, int32_t clear,
                           void *stream) {
    TRY(check_shape(s));
    TRY(check_tokens(T));
    const int E = s->n_experts, k = s->top_k;
    TRY(check_ptr(counts, (size_t)E * 4, 4, "counts"));
    if (T > 0) TRY(check_ptr(topk_ids, (size_t)T * k * 4, 4, "topk_ids"));
    if (T == 0 && !clear) return ok();
    TRY(hip_status(moe::launch_count_picks(topk_ids, T * k, E, counts, clear != 0, static_cast<hipStream_t>(stream)),
                   "pick count launch"));
    return ok();
}

moe_status moe_residency_plan(const moe_shape *s, int32_t *slot_host, int32_t n_hot, int32_t n_cold, double *score,
                              const int32_t *counts_host, double decay, double threshold, double min_score,
                              int32_t max_swaps, int32_t *pairs_out, int32_t *n_pairs_out) {
    TRY(check_shape(s));
    if (!score || !counts_host || !pairs_out || !n_pairs_out)
        return fail(MOE_ERR_INVALID_ARG, "score, counts_host, pairs_out and n_pairs_out must not be NULL");
    *n_pairs_out = 0;
    TRY(moe_residency_check(s, slot_host, n_hot, n_cold));
    if (!(decay >= 0.0 && decay <= 1.0)) return fail(MOE_ERR_INVALID_ARG, "decay %g outside [0, 1]", decay);
    if (!(threshold > 0.0) || !std::isfinite(threshold))
        return fail(MOE_ERR_INVALID_ARG, "threshold %g must be positive and finite", threshold);
    if (!(min_score >= 0.0) || !std::isfinite(min_score))
        return fail(MOE_ERR_INVALID_ARG, "min_score %g must be >= 0 and finite", min_score);
    if (max_swaps < 0 || max_swaps > MOE_MAX_SWAPS)
        return fail(MOE_ERR_INVALID_ARG, "max_swaps %d outside [0, %d]", max_swaps, MOE_MAX_SWAPS);
    const int E = s->n_experts;
    for (int e = 0; e < E; ++e) {
        if (!(score[e] >= 0.0) || !std::isfinite(score[e]))
            return fail(MOE_ERR_INVALID_ARG, "score[%d] = %g must be >= 0 and finite", e, score[e]);
        if (counts_host[e] < 0) return fail(MOE_ERR_INVALID_ARG, "counts_host[%d] = %d is negative", e, counts_host[e]);
    }
    *n_pairs_out = moe::plan_swaps(E, slot_host, score, counts_host, decay, threshold, min_score, max_swaps, pairs_out);
    return ok();
}

moe_status moe_residency_swap(const moe_shape *s, const moe_residency *r, const int32_t *pairs, int32_t n_pairs,
                              void *stream) {
    TRY(check_shape(s));
    if (n_pairs < 0 || n_pairs > MOE_MAX_SWAPS)
        return fail(MOE_ERR_INVALID_ARG, "n_pairs %d outside [0, %d]", n_pairs, MOE_MAX_SWAPS);
    TRY(check_residency(s, r));
    if (n_pairs == 0) return ok();
    if (!pairs) return fail(MOE_ERR_INVALID_ARG, "pairs is NULL");
    if (r->n_hot == 0 || r->n_cold == 0) return fail(MOE_ERR_BAD_RESIDENCY, "a swap needs hot and cold experts");
    if (direct_read(r))
        return fail(MOE_ERR_BAD_RESIDENCY, "direct read (scratch == host_cold) has no staging area for a swap");
    const int E = s->n_experts;
    static thread_local unsigned char used[moe::kMaxExperts];
    memset(used, 0, sizeof(used));
    moe::SwapList l{};
    l.n = n_pairs;
    for (int p = 0; p < n_pairs; ++p) {
        const int32_t c = pairs[2 * p], h = pairs[2 * p + 1];
        if (c < 0 || c >= E || h < 0 || h >= E)
            return fail(MOE_ERR_INVALID_ARG, "pair %d: expert outside [0, %d)", p, E);
        if (used[c] || used[h] || c == h)
            return fail(MOE_ERR_INVALID_ARG, "pair %d: expert %d or %d appears twice in the list", p, c, h);
        used[c] = used[h] = 1;
        l.cold[p] = c;
        l.hot[p] = h;
    }
    const size_t B = moe::BlobLayout::make(s->hidden, s->inter).bytes;
    TRY(hip_status(moe::launch_residency_swap(const_cast<int32_t *>(r->slot), const_cast<uint8_t *>(r->hot_base),
                                              const_cast<uint8_t *>(r->host_cold), r->scratch, B, E, r->n_hot,
                                              r->n_cold, l, static_cast<hipStream_t>(stream)),
                   "residency swap launch"));
    return ok();
}

moe_status moe_fingerprint(const moe_shape *s, const moe_residency *r, const int32_t *experts, int32_t n,
                           uint64_t *out, void *stream) {
    TRY(check_shape(s));
    if (n < 0 || n > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "n %d outside [0, 2^20]", n);
    TRY(check_residency(s, r));
    if (n == 0) return ok();
    TRY(check_ptr(experts, (size_t)n * 4, 4, "experts"));
    TRY(check_ptr(out, (size_t)n * 8, 8, "out"));
    const size_t B = moe::BlobLayout::make(s->hidden, s->inter).bytes;
    TRY(hip_status(moe::launch_fingerprint(experts, n, r->slot, r->hot_base, r->host_cold, B, s->n_experts, r->n_hot,
                                           r->n_cold, out, static_cast<hipStream_t>(stream)),
                   "fingerprint launch"));
    return ok();
}

moe_status moe_probe_read(const void *src, size_t bytes, int32_t loads_per_thread, uint32_t *sink, void *stream) {
    if (bytes == 0 || bytes % 16 || bytes > ((size_t)1 << 40))
        return fail(MOE_ERR_INVALID_ARG, "bytes %zu must be a positive multiple of 16", bytes);
    if (loads_per_thread != 1 && loads_per_thread != 2 && loads_per_thread != 4 && loads_per_thread != 8 &&
        loads_per_thread != 16)
        return fail(MOE_ERR_INVALID_ARG, "loads_per_thread %d must be 1, 2, 4, 8 or 16", loads_per_thread);
    TRY(check_ptr(src, bytes, 16, "src"));
    TRY(check_ptr(sink, 4, 4, "sink"));
    TRY(hip_status(moe::launch_probe_read(src, bytes, loads_per_thread, sink, static_cast<hipStream_t>(stream)),
                   "probe launch"));
    return ok();
}

moe_status moe_probe_mfma(int32_t kind, int32_t iters, uint32_t *sink, void *stream) {
    if (kind < 0 || kind > 4) return fail(MOE_ERR_INVALID_ARG, "kind %d must be 0..4", kind);
    if (iters < 1 || iters > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "iters %d must be 1..2^20", iters);
    TRY(check_ptr(sink, 4, 4, "sink"));
    int dev = 0, cus = 0;
    TRY(hip_status(hipGetDevice(&dev), "current device"));
    TRY(hip_status(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "compute unit count"));
    TRY(hip_status(moe::launch_probe_mfma(kind, iters, cus, sink, static_cast<hipStream_t>(stream)), "probe launch"));
    return ok();
}

}  // extern "C"
