// C ABI of the MoE layer library: argument checks, workspace layout, kernel dispatch.
// The interface and its contract are documented in include/moe.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/moe.h"
#include "moe_launch.hpp"

namespace moe {
// Workspace of moe_layer_forward_static: each GPU the library runs on holds its own copy until the
// process ends.  Host code never passes this name to a kernel (on the host it names a stand-in,
// not device memory): it takes the array's device address once per device from
// hipGetSymbolAddress, with that device current, and uses that address from then on.
__device__ __align__(256) uint8_t scratch[MOE_STATIC_WORKSPACE_BYTES];
}  // namespace moe

namespace {

using namespace moe;

constexpr size_t ALIGN = 256;
constexpr int MAX_T = 32768;
constexpr int SMALL_T_SELECT = 64;    // top-k inside the single-workgroup permute up to this T

size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr uint32_t PREFILL_FLAGS = MOE_F_PREFILL_I8 | MOE_F_PREFILL_FP8;

bool is_fp8(int fmt) { return fmt == MOE_W_FP8_ROW || fmt == MOE_W_FP8_ROW_TILED; }

struct Layout {
    size_t logits = 0, topk_idx = 0, topk_w = 0;
    size_t counts = 0, offsets = 0, perm = 0, inv = 0, slots = 0, n_active = 0, tile_off = 0, scratch = 0;
    size_t tiles = 0;
    size_t h = 0, ybuf = 0, gmask = 0;
    size_t xq = 0, sx = 0, hq = 0, sh = 0;
    size_t total = 0;
};

// Region offsets inside the workspace.  with_route: the call computes the router too.
// S shared experts add S * T pair rows after the T * k routed ones (h, y, the permuted order) and
// S slot records after the E routed ones.
Layout make_layout(int T, int k, int E, int S, int d, int d_ff, int fmt, uint32_t flags, bool with_route)
{
    Layout L;
    size_t o = 0;
    const size_t P = (size_t)T * k;
    const size_t PS = P + (size_t)S * T;         // routed and shared pair rows
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += up(bytes ? bytes : 1);
        return at;
    };
    if (with_route) {
        L.logits = take(sizeof(double) * T * E);
        L.topk_idx = take(sizeof(int32_t) * P);
        L.topk_w = take(sizeof(float) * P);
    }
    L.counts = take(sizeof(int32_t) * E);
    L.offsets = take(sizeof(int32_t) * (E + 1));
    L.perm = take(sizeof(int32_t) * PS);
    L.inv = take(sizeof(int32_t) * P);
    L.slots = take(sizeof(int4) * SLOT_INT4 * (E + S));
    L.n_active = take(sizeof(int32_t));
    L.tile_off = take(sizeof(int32_t) * (E + 1));
    L.scratch = take(sizeof(int32_t) * (size_t)permute_scratch_ints((int)P, E));
    L.tiles = take(sizeof(int4) * (size_t)prefill_tile_bound((int)PS, E + S));
    L.h = take(sizeof(float) * PS * d_ff);    // fp32 h, or the two bf16 planes of h
    if (fmt == MOE_W_E2M1_G16) {
        L.ybuf = take(sizeof(float) * PS * (size_t)e2m1_down_chunks(d_ff, T) * d);
        L.gmask = take(e2m1_mask_bytes(E, S, d_ff));
    } else {
        L.ybuf = take(sizeof(float) * PS * d);
    }
    if (flags & PREFILL_FLAGS) {
        L.xq = take((size_t)T * d);
        L.sx = take(sizeof(float) * T);
        L.hq = take(prefill_h_tiles_bytes((int)PS, E + S, d_ff));
        L.sh = take(sizeof(float) * PS);
    }
    L.total = o;
    return L;
}

moe_status check_experts(const moe_experts *ex, int act, uint32_t flags)
{
    if (!ex) return MOE_EINVAL;
    if (ex->fmt < MOE_W_Q8_0 || ex->fmt > MOE_W_FP8_ROW_TILED) return MOE_EINVAL;
    if (act != MOE_ACT_SWIGLU && act != MOE_ACT_RELU2) return MOE_EINVAL;
    if (ex->E < 1 || ex->E > MAX_E) return MOE_EINVAL;
    if (ex->n_shared < 0 || ex->n_shared > MAX_SHARED) return MOE_EINVAL;
    if (ex->d_model < 64 || ex->d_model > 16384 || ex->d_model % 64) return MOE_EINVAL;
    if (ex->d_ff < 32 || ex->d_ff > 16384 || ex->d_ff % 32) return MOE_EINVAL;
    if (ex->fmt != MOE_W_E2M1_G16 && ex->d_ff % 64) return MOE_EINVAL;
    if (flags & ~(uint32_t)(MOE_F_ZERO_SKIP | PREFILL_FLAGS)) return MOE_EINVAL;
    if ((flags & PREFILL_FLAGS) == PREFILL_FLAGS) return MOE_EINVAL;
    if ((flags & MOE_F_ZERO_SKIP) && ex->fmt != MOE_W_E2M1_G16) return MOE_EUNSUPPORTED;
    if ((flags & MOE_F_PREFILL_I8) && (ex->fmt == MOE_W_E2M1_G16 || is_fp8(ex->fmt) || act != MOE_ACT_SWIGLU))
        return MOE_EUNSUPPORTED;
    // E4M3 experts run on the fp8 prefill path only, and that path on them only
    if (is_fp8(ex->fmt) != ((flags & MOE_F_PREFILL_FP8) != 0)) return MOE_EUNSUPPORTED;
    if ((flags & MOE_F_PREFILL_FP8) && act != MOE_ACT_SWIGLU) return MOE_EUNSUPPORTED;
    return MOE_OK;
}

moe_status check_expert_ptrs(const moe_experts *ex)
{
    if (!aligned16(ex->gate_up) || !aligned16(ex->gate_up_scales) || !aligned16(ex->down) ||
        !aligned16(ex->down_scales))
        return MOE_EINVAL;
    return MOE_OK;
}

moe_status check_tk(int T, int k, int E)
{
    if (T < 1 || T > MAX_T) return MOE_EINVAL;
    if (k < 1 || k > E || k > MAX_K) return MOE_EINVAL;
    return MOE_OK;
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

ExpertsDev dev_view(const moe_experts *ex)
{
    return ExpertsDev{ex->fmt, ex->E, ex->n_shared, ex->d_model, ex->d_ff, ex->gate_up, ex->gate_up_scales,
                      ex->down, ex->down_scales};
}

PermuteOut permute_view(void *ws, const Layout &L)
{
    return PermuteOut{at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.perm),
                      at<int32_t>(ws, L.inv),    at<int4>(ws, L.slots),      at<int32_t>(ws, L.n_active),
                      at<int32_t>(ws, L.tile_off), at<int32_t>(ws, L.scratch), at<int4>(ws, L.tiles)};
}

// Steps 3-5 once the permutation is in the workspace.
moe_status run_experts(const void *x, int xtype, int T, int k, const moe_experts *ex, int act,
                       uint32_t flags, const int32_t *topk_idx, const float *topk_w, float *out, void *ws,
                       const Layout &L, hipStream_t s, const double *route_logits = nullptr,
                       int32_t *route_idx = nullptr, float *route_w = nullptr)
{
    const ExpertsDev dv = dev_view(ex);
    const PermuteOut po = permute_view(ws, L);
    float *h = at<float>(ws, L.h);
    hipError_t err;
    if (flags & PREFILL_FLAGS) {
        int8_t *xq = at<int8_t>(ws, L.xq), *hq = at<int8_t>(ws, L.hq);
        float *sx = at<float>(ws, L.sx), *sh = at<float>(ws, L.sh), *ybuf = at<float>(ws, L.ybuf);
        const bool fp8 = (flags & MOE_F_PREFILL_FP8) != 0;
        if ((err = launch_quantize_rows(x, xtype, T, ex->d_model, xq, sx, true, fp8, s)) != hipSuccess)
            return MOE_EHIP;
        if ((err = launch_ggemm_gateup_i8(xq, sx, T, k, dv, po, h, s)) != hipSuccess) return MOE_EHIP;
        if ((err = launch_quantize_h_tiles(h, T, k, ex->E, ex->n_shared, ex->d_ff, po, hq, sh, fp8, s)) !=
            hipSuccess)
            return MOE_EHIP;
        if ((err = launch_ggemm_down_i8(hq, sh, T, k, dv, po, ybuf, s)) != hipSuccess) return MOE_EHIP;
        return from_hip(launch_combine_rows(ybuf, po.inv, topk_w, T, k, ex->d_model, 1, ex->n_shared, out, s));
    }
    // route_logits: the first expert kernel's blocks select the experts themselves (no permute
    // step before them)
    const RouteIn ri{route_logits, ex->E, ex->n_shared, route_idx, route_w, po.perm, po.inv, po.slots, po.n_active};
    if (ex->fmt == MOE_W_E2M1_G16) {
        const int nchunk = e2m1_down_chunks(ex->d_ff, T);
        float *partial = at<float>(ws, L.ybuf);
        uint8_t *gmask = at<uint8_t>(ws, L.gmask);
        if ((err = launch_up_e2m1(x, xtype, T, k, dv, act, po, h, ri, gmask, s)) != hipSuccess) return MOE_EHIP;
        if ((err = launch_down_e2m1(h, dv, T, k, (flags & MOE_F_ZERO_SKIP) != 0, po, partial, nchunk, gmask,
                                    s)) != hipSuccess)
            return MOE_EHIP;
        return from_hip(launch_combine_rows(partial, po.inv, topk_w, T, k, ex->d_model, nchunk, ex->n_shared, out, s));
    }
    uint16_t *h_hi = reinterpret_cast<uint16_t *>(h);
    uint16_t *h_lo = h_hi + ((size_t)T * k + (size_t)ex->n_shared * T) * ex->d_ff;   // after every pair row
    if ((err = launch_gateup_int8(x, xtype, T, k, dv, act, po, h_hi, h_lo, ri, s)) != hipSuccess)
        return MOE_EHIP;
    return from_hip(launch_down_int8(h_hi, h_lo, dv, T, k, po, topk_idx, topk_w, out, at<float>(ws, L.ybuf), s));
}

// Checks of moe_layer_forward's arguments other than the workspace.
moe_status check_layer_args(const void *x, int xtype, int T, const float *w_router, const float *router_bias,
                            const moe_experts *ex, int k, int act, uint32_t flags, const float *out,
                            const int32_t *topk_idx_out, const float *topk_w_out)
{
    moe_status st = check_experts(ex, act, flags);
    if (st != MOE_OK) return st;
    if (check_tk(T, k, ex->E) != MOE_OK) return MOE_EINVAL;
    if (xtype != MOE_X_F32 && xtype != MOE_X_BF16) return MOE_EINVAL;
    if (check_expert_ptrs(ex) != MOE_OK) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(out)) return MOE_EINVAL;
    if (router_bias && !aligned16(router_bias)) return MOE_EINVAL;
    if ((topk_idx_out && !aligned16(topk_idx_out)) || (topk_w_out && !aligned16(topk_w_out)))
        return MOE_EINVAL;
    return MOE_OK;
}

// ---- the allocation-free variant of moe_layer_forward (moe_layer_forward_static)
// Its workspace is the file-scope device array moe::scratch at the top of this file.

constexpr int MAX_DEVICES = 64;
std::atomic<void *> g_scratch_ptr[MAX_DEVICES];
std::mutex g_scratch_mu;

// The device the work of `s` runs on.
hipError_t stream_device(hipStream_t s, int *dev)
{
    if (s == nullptr) return hipGetDevice(dev);
    hipDevice_t d;
    const hipError_t e = hipStreamGetDevice(s, &d);
    *dev = static_cast<int>(d);
    return e;
}

// The address of `scratch` on device `dev` (looked up on the first call for that device).
moe_status scratch_on(int dev, void **out)
{
    if (dev < 0 || dev >= MAX_DEVICES) return MOE_EHIP;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess) return MOE_EHIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_EHIP;
            void *q = nullptr;
            const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_EHIP;
            if (e != hipSuccess || q == nullptr) return MOE_EHIP;
            g_scratch_ptr[dev].store(q, std::memory_order_release);
            p = q;
        }
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_str(int32_t status)
{
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported format/activation/flag combination";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
    case MOE_ESCRATCH:
        return "MOE_ESCRATCH: the call needs more workspace than the static buffer of "
               "moe_layer_forward_static holds (MOE_STATIC_WORKSPACE_BYTES)";
    default: return "unknown moe_status";
    }
}

size_t moe_workspace_bytes(int32_t T, int32_t k, const moe_experts *ex, int32_t act, uint32_t flags)
{
    if (check_experts(ex, act, flags) != MOE_OK || check_tk(T, k, ex->E) != MOE_OK) return 0;
    return make_layout(T, k, ex->E, ex->n_shared, ex->d_model, ex->d_ff, ex->fmt, flags, true).total;
}

size_t moe_route_workspace_bytes(int32_t T, int32_t E)
{
    if (T < 1 || T > MAX_T || E < 1 || E > MAX_E) return 0;
    return up(sizeof(double) * (size_t)T * E);
}

moe_status moe_route(const void *x, int32_t xtype, int32_t T, int32_t d_model,
                     const float *w_router, const float *router_bias, int32_t E, int32_t k,
                     int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream)
{
    if (xtype != MOE_X_F32 && xtype != MOE_X_BF16) return MOE_EINVAL;
    if (E < 1 || E > MAX_E) return MOE_EINVAL;
    if (check_tk(T, k, E) != MOE_OK) return MOE_EINVAL;
    if (d_model < 64 || d_model > 16384 || d_model % 64) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_idx) || !aligned16(topk_w) ||
        !aligned16(ws))
        return MOE_EINVAL;
    if (router_bias && !aligned16(router_bias)) return MOE_EINVAL;
    if (ws_bytes < moe_route_workspace_bytes(T, E)) return MOE_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    double *logits = static_cast<double *>(ws);
    hipError_t err = launch_router_logits(x, xtype, T, d_model, w_router, router_bias, E, logits, s);
    if (err != hipSuccess) return MOE_EHIP;
    return from_hip(launch_topk(logits, T, E, k, topk_idx, topk_w, s));
}

moe_status moe_permute(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv, void *stream)
{
    if (E < 1 || E > MAX_E || check_tk(T, k, E) != MOE_OK) return MOE_EINVAL;
    if (!aligned16(topk_idx) || !aligned16(counts) || !aligned16(offsets) || !aligned16(perm) ||
        !aligned16(inv))
        return MOE_EINVAL;
    PermuteOut po{counts, offsets, perm, inv, nullptr, nullptr, nullptr, nullptr, nullptr};
    return from_hip(launch_select_permute(nullptr, topk_idx, T, k, E, nullptr, nullptr, po, 0, 0,
                                          static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const void *x, int32_t xtype, int32_t T, const float *w_router,
                             const float *router_bias, const moe_experts *ex, int32_t k,
                             int32_t act, uint32_t flags, float *out, int32_t *topk_idx_out,
                             float *topk_w_out, void *ws, size_t ws_bytes, void *stream)
{
    moe_status st = check_layer_args(x, xtype, T, w_router, router_bias, ex, k, act, flags, out, topk_idx_out,
                                     topk_w_out);
    if (st != MOE_OK) return st;
    if (!aligned16(ws)) return MOE_EINVAL;
    const Layout L = make_layout(T, k, ex->E, ex->n_shared, ex->d_model, ex->d_ff, ex->fmt, flags, true);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    double *logits = at<double>(ws, L.logits);
    int32_t *idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.topk_idx);
    float *w = topk_w_out ? topk_w_out : at<float>(ws, L.topk_w);
    const PermuteOut po = permute_view(ws, L);
    hipError_t err = launch_router_logits(x, xtype, T, ex->d_model, w_router, router_bias, ex->E,
                                          logits, s);
    if (err != hipSuccess) return MOE_EHIP;
    const int BM = (flags & PREFILL_FLAGS) ? prefill_tile_rows() : 0;
    const bool route_in_experts = ex->fmt == MOE_W_E2M1_G16 ? up_e2m1_can_route(T, k, ex->E, ex->d_model)
                                                            : gateup_can_route(T, k, ex->E);
    if (!(flags & PREFILL_FLAGS) && route_in_experts)
        return run_experts(x, xtype, T, k, ex, act, flags, idx, w, out, ws, L, s, logits, idx, w);
    if (T <= SMALL_T_SELECT) {
        err = launch_select_permute(logits, nullptr, T, k, ex->E, idx, w, po, BM, ex->n_shared, s);
    } else {
        err = launch_topk(logits, T, ex->E, k, idx, w, s);
        if (err == hipSuccess)
            err = launch_select_permute(nullptr, idx, T, k, ex->E, nullptr, nullptr, po, BM, ex->n_shared, s);
    }
    if (err != hipSuccess) return MOE_EHIP;
    return run_experts(x, xtype, T, k, ex, act, flags, idx, w, out, ws, L, s);
}

moe_status moe_layer_forward_static(const void *x, int32_t xtype, int32_t T, const float *w_router,
                                    const float *router_bias, const moe_experts *ex, int32_t k, int32_t act,
                                    uint32_t flags, float *out, int32_t *topk_idx_out, float *topk_w_out,
                                    void *stream)
{
    // the same checks as moe_layer_forward, then the size against the static buffer, before any
    // device work or lookup
    moe_status st = check_layer_args(x, xtype, T, w_router, router_bias, ex, k, act, flags, out, topk_idx_out,
                                     topk_w_out);
    if (st != MOE_OK) return st;
    const size_t need = make_layout(T, k, ex->E, ex->n_shared, ex->d_model, ex->d_ff, ex->fmt, flags, true).total;
    if (need > MOE_STATIC_WORKSPACE_BYTES) return MOE_ESCRATCH;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    if (stream_device(s, &dev) != hipSuccess) return MOE_EHIP;
    void *ws = nullptr;
    if ((st = scratch_on(dev, &ws)) != MOE_OK) return st;
    return moe_layer_forward(x, xtype, T, w_router, router_bias, ex, k, act, flags, out, topk_idx_out, topk_w_out,
                             ws, MOE_STATIC_WORKSPACE_BYTES, stream);
}

moe_status moe_experts_forward(const void *x, int32_t xtype, int32_t T, const int32_t *topk_idx,
                               const float *topk_w, const moe_experts *ex, int32_t k, int32_t act,
                               uint32_t flags, float *out, void *ws, size_t ws_bytes, void *stream)
{
    moe_status st = check_experts(ex, act, flags);
    if (st != MOE_OK) return st;
    if (check_tk(T, k, ex->E) != MOE_OK) return MOE_EINVAL;
    if (xtype != MOE_X_F32 && xtype != MOE_X_BF16) return MOE_EINVAL;
    if (check_expert_ptrs(ex) != MOE_OK) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(topk_idx) || !aligned16(topk_w) || !aligned16(out) ||
        !aligned16(ws))
        return MOE_EINVAL;
    const Layout L = make_layout(T, k, ex->E, ex->n_shared, ex->d_model, ex->d_ff, ex->fmt, flags, false);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const PermuteOut po = permute_view(ws, L);
    const int BM = (flags & PREFILL_FLAGS) ? prefill_tile_rows() : 0;
    hipError_t err = launch_select_permute(nullptr, topk_idx, T, k, ex->E, nullptr, nullptr, po, BM,
                                           ex->n_shared, s);
    if (err != hipSuccess) return MOE_EHIP;
    return run_experts(x, xtype, T, k, ex, act, flags, topk_idx, topk_w, out, ws, L, s);
}

moe_status moe_read_intermediates(int32_t T, int32_t k, const moe_experts *ex, int32_t act, uint32_t flags,
                                  int32_t with_router, const void *ws, size_t ws_bytes, float *h, void *hq,
                                  float *sh, void *stream)
{
    moe_status st = check_experts(ex, act, flags);
    if (st != MOE_OK) return st;
    if (check_tk(T, k, ex->E) != MOE_OK) return MOE_EINVAL;
    if (!aligned16(ws) || !aligned16(h)) return MOE_EINVAL;
    const bool prefill = (flags & PREFILL_FLAGS) != 0;
    if (prefill != (hq != nullptr) || prefill != (sh != nullptr)) return MOE_EINVAL;
    if (prefill && (!aligned16(hq) || !aligned16(sh))) return MOE_EINVAL;
    const Layout L = make_layout(T, k, ex->E, ex->n_shared, ex->d_model, ex->d_ff, ex->fmt, flags, with_router != 0);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *w = const_cast<void *>(ws);
    const PermuteOut po = permute_view(w, L);
    const int P = T * k, rows = P + ex->n_shared * T;
    const float *h32 = nullptr;
    const uint16_t *hh = nullptr, *hl = nullptr;
    if (prefill || ex->fmt == MOE_W_E2M1_G16) {
        h32 = at<float>(w, L.h);
    } else {                                          // int8 decode: two bf16 planes
        hh = at<uint16_t>(w, L.h);
        hl = hh + (size_t)rows * ex->d_ff;
    }
    hipError_t err = launch_unpermute_h(h32, hh, hl, po.perm, P, rows, ex->d_ff, h, s);
    if (err == hipSuccess && prefill)
        err = launch_untile_hq(at<int8_t>(w, L.hq), at<float>(w, L.sh), po, ex->E,
                               prefill_tile_bound(rows, ex->E + ex->n_shared), P, ex->d_ff,
                               static_cast<int8_t *>(hq), sh, s);
    return from_hip(err);
}

moe_status moe_repack_experts(const moe_experts *src, int32_t act, const moe_experts *dst,
                              void *stream)
{
    if (!src || !dst) return MOE_EINVAL;
    if (src->fmt != MOE_W_Q8_0 && src->fmt != MOE_W_I8_ROW && src->fmt != MOE_W_FP8_ROW) return MOE_EINVAL;
    const int want = src->fmt == MOE_W_Q8_0 ? MOE_W_Q8_0_TILED
                     : src->fmt == MOE_W_I8_ROW ? MOE_W_I8_ROW_TILED : MOE_W_FP8_ROW_TILED;
    if (dst->fmt != want || dst->E != src->E || dst->n_shared != src->n_shared ||
        dst->d_model != src->d_model || dst->d_ff != src->d_ff)
        return MOE_EINVAL;
    const uint32_t src_flags = is_fp8(src->fmt) ? (uint32_t)MOE_F_PREFILL_FP8 : 0u;
    if (check_experts(src, act, src_flags) != MOE_OK || check_expert_ptrs(src) != MOE_OK ||
        check_expert_ptrs(dst) != MOE_OK)
        return MOE_EINVAL;
    if (src->gate_up == dst->gate_up || src->down == dst->down) return MOE_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int E = src->E + src->n_shared, d = src->d_model, dff = src->d_ff;   // every expert array
    const int M = act == MOE_ACT_SWIGLU ? 2 : 1;
    const bool q8 = src->fmt == MOE_W_Q8_0;
    const auto *gsrc = static_cast<const int8_t *>(src->gate_up);
    const auto *dsrc = static_cast<const int8_t *>(src->down);
    auto *gdst = static_cast<int8_t *>(const_cast<void *>(dst->gate_up));
    auto *ddst = static_cast<int8_t *>(const_cast<void *>(dst->down));
    hipError_t err = launch_repack_tiled(
        gsrc, q8 ? static_cast<const uint16_t *>(src->gate_up_scales) : nullptr, E, M * dff, d, M, gdst,
        q8 ? static_cast<uint16_t *>(const_cast<void *>(dst->gate_up_scales)) : nullptr, s);
    if (err == hipSuccess)
        err = launch_repack_tiled(
            dsrc, q8 ? static_cast<const uint16_t *>(src->down_scales) : nullptr, E, d, dff, 1, ddst,
            q8 ? static_cast<uint16_t *>(const_cast<void *>(dst->down_scales)) : nullptr, s);
    if (err == hipSuccess && !q8) {
        err = hipMemcpyAsync(const_cast<void *>(dst->gate_up_scales), src->gate_up_scales,
                             sizeof(float) * (size_t)E * M * dff, hipMemcpyDeviceToDevice, s);
        if (err == hipSuccess)
            err = hipMemcpyAsync(const_cast<void *>(dst->down_scales), src->down_scales,
                                 sizeof(float) * (size_t)E * d, hipMemcpyDeviceToDevice, s);
    }
    return from_hip(err);
}

moe_status moe_quantize_rows_i8(const void *v, int32_t xtype, int32_t rows, int32_t cols, int8_t *q,
                                float *scale, void *stream)
{
    if (xtype != MOE_X_F32 && xtype != MOE_X_BF16) return MOE_EINVAL;
    if (rows < 1 || rows > (1 << 24) || cols < 64 || cols > 16384 || cols % 64) return MOE_EINVAL;
    if (!aligned16(v) || !aligned16(q) || !aligned16(scale)) return MOE_EINVAL;
    return from_hip(launch_quantize_rows(v, xtype, rows, cols, q, scale, false, false,
                                         static_cast<hipStream_t>(stream)));
}

moe_status moe_quantize_rows_fp8(const void *v, int32_t xtype, int32_t rows, int32_t cols, uint8_t *q,
                                 float *scale, void *stream)
{
    if (xtype != MOE_X_F32 && xtype != MOE_X_BF16) return MOE_EINVAL;
    if (rows < 1 || rows > (1 << 24) || cols < 64 || cols > 16384 || cols % 64) return MOE_EINVAL;
    if (!aligned16(v) || !aligned16(q) || !aligned16(scale)) return MOE_EINVAL;
    return from_hip(launch_quantize_rows(v, xtype, rows, cols, reinterpret_cast<int8_t *>(q), scale, false, true,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
