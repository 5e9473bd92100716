// C ABI of the Flint MoE layer: host-side validation, workspace carving and
// launch sequencing.  Every check runs before the first launch, so an argument
// error leaves the outputs untouched.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/flint_moe.h"
#include "launch.hpp"

using namespace flint;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by every entry point.  Returns FLINT_OK or an error.
flint_status check_dims(const flint_moe_dims *d)
{
    if (!d) return FLINT_INVALID_ARG;
    if (d->dtype != FLINT_F32 && d->dtype != FLINT_BF16) return FLINT_UNSUPPORTED;
    if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->inter <= 0 || d->shared_inter < 0)
        return FLINT_INVALID_ARG;
    if (d->top_k > d->n_experts) return FLINT_INVALID_ARG;
    if (d->top_k > kMaxTopK || d->n_experts > kMaxExperts) return FLINT_UNSUPPORTED;
    if (d->hidden % 64 || d->inter % 64 || d->shared_inter % 64) return FLINT_UNSUPPORTED;
    if (d->hidden > 8192 || d->inter > 4096 || d->shared_inter > 4096) return FLINT_UNSUPPORTED;
    return FLINT_OK;
}

flint_status check_T(const flint_moe_dims *d, int32_t T)
{
    if (T < 0) return FLINT_INVALID_ARG;
    if ((int64_t)T * d->top_k >= (int64_t)1 << 31) return FLINT_UNSUPPORTED;
    // slot indices times H must fit the kernels' size_t arithmetic; row counts fit int
    if ((int64_t)T * d->top_k * d->hidden >= (int64_t)1 << 40) return FLINT_UNSUPPORTED;
    return FLINT_OK;
}

int elem_bytes(const flint_moe_dims *d) { return d->dtype == FLINT_BF16 ? 2 : 4; }

}  // namespace

namespace flint {

// Compute units of the current device, read once per device (the only state
// the library keeps).  Falls back to 256 (MI355X) if the query fails.
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int list_capacity(int T, int K, int E, int bm)
{
    const long long pairs = (long long)T * K;
    const long long nonempty = pairs < E ? pairs : E;
    return (int)(pairs / bm + nonempty + 1);
}

// The intermediate arrays (h, y) start at a fixed phase within 4 KB against
// the output buffer: 1 KB past it.  The combine reads rows of y while it
// writes the same rows of the output, and its speed depends on where the two
// fall against each other (measured, the Flint layer with the output on a
// 4 KB boundary: T = 16384 combine 121 us at 1 KB, 127 at 512 bytes, 139 at
// 0 and at 2 KB; T = 4096 27 us at 1 KB, 31 at 0).  Sizing (no base) reserves
// the largest padding.
constexpr size_t kPhasePeriod = 4096, kPhaseOffset = 1024;

static Workspace plan_workspace_out(void *base, const void *out, int T, int H, int E, int K, int I, int Is, int eb,
                                    int shared_splits)
{
    Workspace w{};
    const size_t TK = (size_t)T * K;
    const int ntiles = (T + kTopkTile - 1) / kTopkTile;
    const ExpertTiles tiles = expert_tiles_for(T, H, E, K, I, Is, eb == 2);
    int bm1 = tiles.bm1, bm2 = tiles.bm2;
    if (eb == 2 && T <= kMx4MaxT) {
        // room for the lists of the MXFP4 kernels too (one workspace size per dims and T)
        bm1 = std::min(bm1, mx4_bm1());
        bm2 = std::min(bm2, mx4_bm2());
    }
    const int cap1 = list_capacity(T, K, E, bm1);
    const int cap2 = list_capacity(T, K, E, bm2);
    size_t off = 0;
    char *b = (char *)base;
    auto take = [&](size_t bytes) -> void * {
        void *p = b ? (void *)(b + off) : nullptr;
        off += align_up(bytes ? bytes : 1);
        return p;
    };
    auto phase = [&]() {
        if (!b) {
            off += kPhasePeriod;
            return;
        }
        const uintptr_t want = ((uintptr_t)out + kPhaseOffset) % kPhasePeriod;
        off += ((want + kPhasePeriod - ((uintptr_t)b + off) % kPhasePeriod) % kPhasePeriod) / kAlign * kAlign;
    };
    w.logits = (float *)take((size_t)router_splits(T, H, E, eb == 2) * T * E * 4);
    w.hist = (int32_t *)take((size_t)ntiles * E * 4);
    w.tile_base = (int32_t *)take((size_t)ntiles * E * 4);
    w.rank = (int32_t *)take(TK * 4);
    w.topk_idx = (int32_t *)take(TK * 4);
    w.topk_w = (float *)take(TK * 4);
    w.counts = (int32_t *)take((size_t)E * 4);
    w.offsets = (int32_t *)take((size_t)(E + 1) * 4);
    w.sorted_token = (int32_t *)take(TK * 4);
    w.slot_of = (int32_t *)take(TK * 4);
    w.list1 = (int32_t *)take((size_t)cap1 * 8);
    w.list2 = (int32_t *)take((size_t)cap2 * 8);
    w.meta = (int32_t *)take(16);
    phase();
    w.h_sorted = take(TK * I * eb);
    w.h_shared = take((size_t)T * Is * eb);
    phase();
    w.y_sorted = (float *)take(TK * H * 4);
    phase();
    w.y_shared = (float *)take((size_t)shared_splits * T * H * 4);
    if (tiles.tiled && K > 0) w.y_scale = (int8_t *)take((TK + T) * (H / kYScaleCols));
    if (K > 0) w.done = (int32_t *)take(4);
    if (eb == 2 && K > 0 && T <= kFusedMaxT) {  // the fused decode kernel's own state
        w.topk_q = (int32_t *)take((size_t)kFusedQueues * TK * 4);
        w.sync = (int32_t *)take((size_t)kFusedSyncWords * 4);
    }
    w.bytes = off;
    return w;
}

Workspace plan_workspace(void *base, int T, int H, int E, int K, int I, int Is, int eb, int shared_splits)
{
    return plan_workspace_out(base, nullptr, T, H, E, K, I, Is, eb, shared_splits);
}

// On the streaming kernels a shared down item reduces over Is and a routed one
// over I; with Is a multiple of I and up to 64 tokens the shared reduction is
// split into Is / I partial arrays (the combine adds them in order), so that
// every down item of the persistent walk is the same length.  Measured (Flint
// shape): T = 32 down 57.6 -> 55.5 us, T = 8 23.0 -> 22.3 us; at T = 128 the
// extra partial array costs more than the balance gains, at 256 it is even.
constexpr int kMoeSharedSplitT = 64;
static bool fused_ok(const flint_moe_dims *d, int32_t T)
{
    return fused_eligible(T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter, d->dtype == FLINT_BF16);
}

// fused: the layer runs on the fused decode kernel, which cuts the shared
// expert into Is / I slices
int moe_shared_splits(const flint_moe_dims *d, int32_t T, bool mx4, bool fused = false)
{
    if (fused) return d->shared_inter > 0 ? d->shared_inter / d->inter : 1;
    if (T > kMoeSharedSplitT || mx4 || d->shared_inter <= d->inter || d->shared_inter % d->inter) return 1;
    const int s = d->shared_inter / d->inter;
    if (s > 8) return 1;
    const bool bf16 = d->dtype == FLINT_BF16;
    if (!expert_tiles_for(T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter, bf16).stream ||
        !stream_eligible(T, d->hidden, d->inter, d->shared_inter / s))
        return 1;
    return s;
}

}  // namespace flint

extern "C" {

const char *flint_status_string(flint_status s)
{
    switch (s) {
    case FLINT_OK: return "ok";
    case FLINT_INVALID_ARG: return "invalid argument";
    case FLINT_UNSUPPORTED: return "unsupported configuration (refused; there is no fallback path)";
    case FLINT_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FLINT_DEVICE_ERROR: return "device error at launch";
    default: return "unknown status";
    }
}

size_t flint_moe_workspace_bytes(const flint_moe_dims *d, int32_t T)
{
    if (check_dims(d) != FLINT_OK || check_T(d, T) != FLINT_OK) return 0;
    // room for every path a forward call of this shape may take
    int splits = moe_shared_splits(d, T, false);
    if (fused_ok(d, T)) splits = std::max(splits, moe_shared_splits(d, T, false, true));
    return plan_workspace(nullptr, T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter,
                          elem_bytes(d), splits)
        .bytes;
}

static flint_status check_ws(const flint_moe_dims *d, int32_t T, const void *ws, size_t ws_bytes)
{
    const size_t need = flint_moe_workspace_bytes(d, T);
    if (ws_bytes < need) return FLINT_WORKSPACE_TOO_SMALL;
    if (!ws) return FLINT_INVALID_ARG;
    if (((uintptr_t)ws & (kAlign - 1)) != 0) return FLINT_UNSUPPORTED;
    return FLINT_OK;
}

flint_status flint_moe_route(const flint_moe_dims *d, int32_t T, const void *x, const void *router,
                             const float *router_bias, int32_t *topk_idx, float *topk_w, void *ws,
                             size_t ws_bytes, void *stream)
{
    flint_status st = check_dims(d);
    if (st != FLINT_OK) return st;
    if ((st = check_T(d, T)) != FLINT_OK) return st;
    if (T == 0) return FLINT_OK;
    if (!x || !router || !topk_idx || !topk_w) return FLINT_INVALID_ARG;
    if (!aligned16(x) || !aligned16(router) || !aligned16(topk_idx) || !aligned16(topk_w) ||
        (router_bias && !aligned16(router_bias)))
        return FLINT_UNSUPPORTED;
    if ((st = check_ws(d, T, ws, ws_bytes)) != FLINT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    Workspace w = plan_workspace(ws, T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter,
                                 elem_bytes(d));
    if (launch_router_logits(d->dtype == FLINT_BF16, x, T, d->hidden, router, router_bias, d->n_experts,
                             w.logits, s) != hipSuccess)
        return FLINT_DEVICE_ERROR;
    DispatchArgs a{};
    a.T = T;
    a.E = d->n_experts;
    a.K = d->top_k;
    a.logits = w.logits;
    a.logit_splits = router_splits(T, d->hidden, d->n_experts, d->dtype == FLINT_BF16);
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.compute_topk = true;
    a.dispatch = false;
    if (launch_topk_dispatch(a, s) != hipSuccess) return FLINT_DEVICE_ERROR;
    return FLINT_OK;
}

static DispatchArgs dispatch_args(const flint_moe_dims *d, int32_t T, const Workspace &w)
{
    DispatchArgs a{};
    const ExpertTiles tiles = expert_tiles_for(T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter,
                                               d->dtype == FLINT_BF16);
    a.T = T;
    a.E = d->n_experts;
    a.K = d->top_k;
    a.hist = w.hist;
    a.tile_base = w.tile_base;
    a.rank = w.rank;
    a.list1 = w.list1;
    a.list2 = w.list2;
    a.meta = w.meta;
    a.bm1 = tiles.bm1;
    a.bm2 = tiles.bm2;
    a.dispatch = true;
    return a;
}

flint_status flint_moe_dispatch(const flint_moe_dims *d, int32_t T, const int32_t *topk_idx,
                                int32_t *counts, int32_t *offsets, int32_t *sorted_token, int32_t *slot_of,
                                void *ws, size_t ws_bytes, void *stream)
{
    flint_status st = check_dims(d);
    if (st != FLINT_OK) return st;
    if ((st = check_T(d, T)) != FLINT_OK) return st;
    if (!counts || !offsets) return FLINT_INVALID_ARG;
    if (T > 0 && (!topk_idx || !sorted_token || !slot_of)) return FLINT_INVALID_ARG;
    if (!aligned16(counts) || !aligned16(offsets) ||
        (T > 0 && (!aligned16(topk_idx) || !aligned16(sorted_token) || !aligned16(slot_of))))
        return FLINT_UNSUPPORTED;
    if ((st = check_ws(d, T, ws, ws_bytes)) != FLINT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        // every count and offset is zero (a fill kernel, not a memset node, so
        // that the call can be captured in a graph)
        if (launch_fill_i32(counts, d->n_experts, 0, s) != hipSuccess) return FLINT_DEVICE_ERROR;
        if (launch_fill_i32(offsets, d->n_experts + 1, 0, s) != hipSuccess) return FLINT_DEVICE_ERROR;
        return FLINT_OK;
    }
    Workspace w = plan_workspace(ws, T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter,
                                 elem_bytes(d));
    DispatchArgs a = dispatch_args(d, T, w);
    a.topk_idx = const_cast<int32_t *>(topk_idx);
    a.compute_topk = false;
    a.counts = counts;
    a.offsets = offsets;
    a.sorted_token = sorted_token;
    a.slot_of = slot_of;
    if (launch_topk_dispatch(a, s) != hipSuccess) return FLINT_DEVICE_ERROR;
    return FLINT_OK;
}

flint_status flint_moe_forward(const flint_moe_dims *d, int32_t T, const void *x, const flint_moe_weights *wt,
                               void *out, flint_dtype out_dtype, int32_t *topk_idx_out, float *topk_w_out,
                               void *ws, size_t ws_bytes, void *stream)
{
    return flint_moe_forward_profiled(d, T, x, wt, out, out_dtype, topk_idx_out, topk_w_out, ws, ws_bytes, stream,
                                      nullptr);
}

}  // extern "C"

// The layer's launches once the arguments are checked: router, top-k +
// dispatch, expert stages, combine.  `e` arrives with the weight pointers set.
static flint_status launch_layer(const flint_moe_dims *d, int32_t T, const void *x, const void *router,
                                 const float *router_bias, ExpertArgs e, void *out, flint_dtype out_dtype,
                                 int32_t *topk_idx_out, float *topk_w_out, void *ws, void *stream,
                                 void *const *events, bool fused = false)
{
    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = d->dtype == FLINT_BF16;
    const int shared_splits = moe_shared_splits(d, T, e.mx4, fused);
    Workspace w = plan_workspace_out(ws, out, T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter,
                                     elem_bytes(d), shared_splits);
    // stage marks: router, top-k + dispatch, gate/up, down, combine
    Marks marks[5];
    if (events)
        for (int i = 0; i < 5; ++i) marks[i] = Marks{(hipEvent_t)events[2 * i], (hipEvent_t)events[2 * i + 1]};
    const ExpertTiles tiles = expert_tiles_for(T, d->hidden, d->n_experts, d->top_k, d->inter, d->shared_inter,
                                               d->dtype == FLINT_BF16);
    // the router kernel also zeroes the counters of what follows it: the fused
    // decode kernel's, or that of the one-tile top-k + dispatch
    int32_t *const zero = fused ? w.sync : (T <= kTopkTile ? w.done : nullptr);
    if (launch_router_logits(bf16, x, T, d->hidden, router, router_bias, d->n_experts, w.logits, s, marks[0], zero,
                             fused ? kFusedSyncWords : (zero ? 1 : 0)) != hipSuccess)
        return FLINT_DEVICE_ERROR;
    if (fused) {
        // top-k, dispatch, gate/up and down in one launch (stage marks: the
        // kernel is stage 1; stages 2 and 3 are empty), then the combine
        e.bf16 = true;
        e.T = T;
        e.H = d->hidden;
        e.E = d->n_experts;
        e.K = d->top_k;
        e.I = d->inter;
        e.Is = d->shared_inter;
        e.x = x;
        e.sorted_token = w.sorted_token;
        e.offsets = w.offsets;
        e.slot_of = w.slot_of;
        e.topk_w = topk_w_out ? topk_w_out : w.topk_w;
        e.h_sorted = w.h_sorted;
        e.h_shared = w.h_shared;
        e.y_sorted = w.y_sorted;
        e.y_shared = w.y_shared;
        e.shared_splits = shared_splits;
        e.out = out;
        e.out_bf16 = out_dtype == FLINT_BF16;
        e.tiles = tiles;
        e.cus = device_cus();
        e.fail = w.sync + (2 * kFusedQueues + kMaxExperts + kFusedMaxShared) * 32;
        if (launch_fused_decode(e, w.logits, router_splits(T, d->hidden, d->n_experts, bf16),
                                topk_idx_out ? topk_idx_out : w.topk_idx, const_cast<float *>(e.topk_w), w.topk_q,
                                w.sync, w.counts, w.offsets, w.sorted_token, w.slot_of, s,
                                Marks{marks[1].start, marks[1].stop}) != hipSuccess)
            return FLINT_DEVICE_ERROR;
        for (int i = 2; i <= 3; ++i) {
            if (marks[i].start && hipEventRecord(marks[i].start, s) != hipSuccess) return FLINT_DEVICE_ERROR;
            if (marks[i].stop && hipEventRecord(marks[i].stop, s) != hipSuccess) return FLINT_DEVICE_ERROR;
        }
        if (launch_combine(e, s, marks[4]) != hipSuccess) return FLINT_DEVICE_ERROR;
        return FLINT_OK;
    }

    DispatchArgs a = dispatch_args(d, T, w);
    if (e.mx4) {
        a.bm1 = mx4_bm1();
        a.bm2 = mx4_bm2();
    }
    a.logits = w.logits;
    a.logit_splits = router_splits(T, d->hidden, d->n_experts, bf16);
    a.topk_idx = topk_idx_out ? topk_idx_out : w.topk_idx;
    a.topk_w = topk_w_out ? topk_w_out : w.topk_w;
    a.compute_topk = true;
    if (!e.mx4 && tiles.tiled) {
        a.y_scale = w.y_scale;
        a.scale_cols = d->hidden / kYScaleCols;
    }
    a.counts = w.counts;
    a.offsets = w.offsets;
    a.sorted_token = w.sorted_token;
    a.slot_of = w.slot_of;
    a.done = w.done;  // one tile: zeroed by the router kernel above; several: by the top-k kernel
    if (launch_topk_dispatch(a, s, marks[1]) != hipSuccess) return FLINT_DEVICE_ERROR;

    e.bf16 = bf16;
    e.T = T;
    e.H = d->hidden;
    e.E = d->n_experts;
    e.K = d->top_k;
    e.I = d->inter;
    e.Is = d->shared_inter;
    e.x = x;
    e.sorted_token = w.sorted_token;
    e.offsets = w.offsets;
    e.slot_of = w.slot_of;
    e.topk_w = a.topk_w;
    e.list1 = w.list1;
    e.list2 = w.list2;
    e.meta = w.meta;
    e.h_sorted = w.h_sorted;
    e.h_shared = w.h_shared;
    e.y_sorted = w.y_sorted;
    e.y_shared = w.y_shared;
    e.y_scale = w.y_scale;
    e.shared_splits = shared_splits;
    e.out = out;
    e.out_bf16 = out_dtype == FLINT_BF16;
    e.tiles = tiles;
    e.cus = device_cus();
    if (launch_experts(e, s, events ? marks + 2 : nullptr) != hipSuccess) return FLINT_DEVICE_ERROR;
    return FLINT_OK;
}

// Checks shared by both forward entry points: everything but the weights and
// the workspace.
static flint_status check_forward_args(const flint_moe_dims *d, int32_t T, const void *x, const void *router,
                                       const float *router_bias, void *out, flint_dtype out_dtype,
                                       int32_t *topk_idx_out, float *topk_w_out)
{
    flint_status st = check_dims(d);
    if (st != FLINT_OK) return st;
    if ((st = check_T(d, T)) != FLINT_OK) return st;
    if (out_dtype != FLINT_F32 && out_dtype != FLINT_BF16) return FLINT_UNSUPPORTED;
    if (T == 0) return FLINT_OK;
    if (!x || !out || !router) return FLINT_INVALID_ARG;
    if (!aligned16(x) || !aligned16(out) || !aligned16(router)) return FLINT_UNSUPPORTED;
    if (router_bias && !aligned16(router_bias)) return FLINT_UNSUPPORTED;
    if ((topk_idx_out && !aligned16(topk_idx_out)) || (topk_w_out && !aligned16(topk_w_out)))
        return FLINT_UNSUPPORTED;
    return FLINT_OK;
}

static flint_status check_forward(const flint_moe_dims *d, int32_t T, const void *x, const void *router,
                                  const float *router_bias, void *out, flint_dtype out_dtype,
                                  int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes)
{
    const flint_status st =
        check_forward_args(d, T, x, router, router_bias, out, out_dtype, topk_idx_out, topk_w_out);
    if (st != FLINT_OK || T == 0) return st;
    return check_ws(d, T, ws, ws_bytes);
}

// The bf16/float32 weight pointers (after check_dims).
static flint_status check_weights(const flint_moe_dims *d, const flint_moe_weights *wt)
{
    if (!wt->gate || !wt->up || !wt->down) return FLINT_INVALID_ARG;
    const bool has_shared = d->shared_inter > 0;
    if (has_shared && (!wt->shared_gate || !wt->shared_up || !wt->shared_down)) return FLINT_INVALID_ARG;
    if (!aligned16(wt->gate) || !aligned16(wt->up) || !aligned16(wt->down)) return FLINT_UNSUPPORTED;
    if (has_shared && (!aligned16(wt->shared_gate) || !aligned16(wt->shared_up) || !aligned16(wt->shared_down)))
        return FLINT_UNSUPPORTED;
    return FLINT_OK;
}

namespace flint {

// Every check flint_moe_forward makes except the workspace's (used by the
// entry point whose workspace is the library's own static scratch).
flint_status check_forward_call(const flint_moe_dims *d, int32_t T, const void *x, const flint_moe_weights *wt,
                                void *out, flint_dtype out_dtype, int32_t *topk_idx_out, float *topk_w_out)
{
    const flint_status st = check_forward_args(d, T, x, wt ? wt->router : nullptr, wt ? wt->router_bias : nullptr,
                                               out, out_dtype, topk_idx_out, topk_w_out);
    if (st != FLINT_OK || T == 0) return st;
    return check_weights(d, wt);
}

}  // namespace flint

extern "C" {

flint_status flint_moe_forward_profiled(const flint_moe_dims *d, int32_t T, const void *x,
                                        const flint_moe_weights *wt, void *out, flint_dtype out_dtype,
                                        int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                                        void *stream, void *const *events)
{
    flint_status st = check_forward(d, T, x, wt ? wt->router : nullptr, wt ? wt->router_bias : nullptr, out,
                                    out_dtype, topk_idx_out, topk_w_out, ws, ws_bytes);
    if (st != FLINT_OK || T == 0) return st;
    if ((st = check_weights(d, wt)) != FLINT_OK) return st;
    ExpertArgs e{};
    e.gate = wt->gate;
    e.up = wt->up;
    e.down = wt->down;
    e.shared_gate = wt->shared_gate;
    e.shared_up = wt->shared_up;
    e.shared_down = wt->shared_down;
    return launch_layer(d, T, x, wt->router, wt->router_bias, e, out, out_dtype, topk_idx_out, topk_w_out, ws,
                        stream, events);
}

flint_status flint_moe_forward_rmsnorm(const flint_moe_dims *d, int32_t T, const void *x,
                                       const flint_moe_weights *wt, void *out, flint_dtype out_dtype,
                                       void *norm_out_bf16, float eps, int32_t *topk_idx_out, float *topk_w_out,
                                       void *ws, size_t ws_bytes, void *stream, void *const *events)
{
    flint_status st = check_forward(d, T, x, wt ? wt->router : nullptr, wt ? wt->router_bias : nullptr, out,
                                    out_dtype, topk_idx_out, topk_w_out, ws, ws_bytes);
    if (st != FLINT_OK) return st;
    if (d->hidden % 64 || d->hidden > 8192) return FLINT_UNSUPPORTED;
    if (!(eps >= 0.0f)) return FLINT_INVALID_ARG;
    if (T == 0) return FLINT_OK;
    if (!norm_out_bf16) return FLINT_INVALID_ARG;
    if (!aligned16(norm_out_bf16)) return FLINT_UNSUPPORTED;
    const size_t row = (size_t)d->hidden, n_bytes = (size_t)T * row * 2,
                 out_bytes = (size_t)T * row * (out_dtype == FLINT_BF16 ? 2 : 4);
    const uintptr_t n0 = (uintptr_t)norm_out_bf16, o0 = (uintptr_t)out;
    if (n0 < o0 + out_bytes && o0 < n0 + n_bytes) return FLINT_INVALID_ARG;  // overlaps out
    if ((st = check_weights(d, wt)) != FLINT_OK) return st;
    ExpertArgs e{};
    e.gate = wt->gate;
    e.up = wt->up;
    e.down = wt->down;
    e.shared_gate = wt->shared_gate;
    e.shared_up = wt->shared_up;
    e.shared_down = wt->shared_down;
    e.norm_out = (uint16_t *)norm_out_bf16;
    e.norm_eps = eps;
    return launch_layer(d, T, x, wt->router, wt->router_bias, e, out, out_dtype, topk_idx_out, topk_w_out, ws,
                        stream, events);
}

flint_status flint_moe_forward_fused(const flint_moe_dims *d, int32_t T, const void *x, const flint_moe_weights *wt,
                                     void *out, flint_dtype out_dtype, int32_t *topk_idx_out, float *topk_w_out,
                                     void *ws, size_t ws_bytes, void *stream, void *const *events)
{
    flint_status st = check_forward(d, T, x, wt ? wt->router : nullptr, wt ? wt->router_bias : nullptr, out,
                                    out_dtype, topk_idx_out, topk_w_out, ws, ws_bytes);
    if (st != FLINT_OK || T == 0) return st;
    if ((st = check_weights(d, wt)) != FLINT_OK) return st;
    if (!fused_ok(d, T)) return FLINT_UNSUPPORTED;
    ExpertArgs e{};
    e.gate = wt->gate;
    e.up = wt->up;
    e.down = wt->down;
    e.shared_gate = wt->shared_gate;
    e.shared_up = wt->shared_up;
    e.shared_down = wt->shared_down;
    return launch_layer(d, T, x, wt->router, wt->router_bias, e, out, out_dtype, topk_idx_out, topk_w_out, ws,
                        stream, events, true);
}

flint_status flint_moe_forward_mx4(const flint_moe_dims *d, int32_t T, const void *x,
                                   const flint_moe_weights_mx4 *wt, void *out, flint_dtype out_dtype,
                                   int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                                   void *stream, void *const *events)
{
    flint_status st = check_dims(d);
    if (st != FLINT_OK) return st;
    if (d->dtype != FLINT_BF16) return FLINT_UNSUPPORTED;
    if (T > kMx4MaxT || !mx4_eligible(T, d->hidden, d->inter, d->shared_inter)) return FLINT_UNSUPPORTED;
    st = check_forward(d, T, x, wt ? wt->router : nullptr, wt ? wt->router_bias : nullptr, out, out_dtype,
                       topk_idx_out, topk_w_out, ws, ws_bytes);
    if (st != FLINT_OK || T == 0) return st;
    const bool has_shared = d->shared_inter > 0;
    const uint8_t *need[] = {wt->gate_q, wt->gate_s, wt->up_q, wt->up_s, wt->down_q, wt->down_s};
    for (const uint8_t *p : need)
        if (!p) return FLINT_INVALID_ARG;
    const uint8_t *need_shared[] = {wt->shared_gate_q, wt->shared_gate_s, wt->shared_up_q,
                                    wt->shared_up_s,   wt->shared_down_q, wt->shared_down_s};
    if (has_shared)
        for (const uint8_t *p : need_shared)
            if (!p) return FLINT_INVALID_ARG;
    if (!aligned16(wt->gate_q) || !aligned16(wt->up_q) || !aligned16(wt->down_q)) return FLINT_UNSUPPORTED;
    if (has_shared && (!aligned16(wt->shared_gate_q) || !aligned16(wt->shared_up_q) || !aligned16(wt->shared_down_q)))
        return FLINT_UNSUPPORTED;
    ExpertArgs e{};
    e.mx4 = true;
    e.gate = wt->gate_q;
    e.up = wt->up_q;
    e.down = wt->down_q;
    e.gate_s = wt->gate_s;
    e.up_s = wt->up_s;
    e.down_s = wt->down_s;
    e.shared_gate = wt->shared_gate_q;
    e.shared_up = wt->shared_up_q;
    e.shared_down = wt->shared_down_q;
    e.shared_gate_s = wt->shared_gate_s;
    e.shared_up_s = wt->shared_up_s;
    e.shared_down_s = wt->shared_down_s;
    return launch_layer(d, T, x, wt->router, wt->router_bias, e, out, out_dtype, topk_idx_out, topk_w_out, ws,
                        stream, events);
}

}  // extern "C"

namespace {

flint_status check_dense(const flint_dense_dims *d, int32_t T)
{
    if (!d) return FLINT_INVALID_ARG;
    if (d->dtype != FLINT_F32 && d->dtype != FLINT_BF16) return FLINT_UNSUPPORTED;
    if (d->hidden <= 0 || d->inter <= 0 || T < 0) return FLINT_INVALID_ARG;
    if (d->hidden % 64 || d->inter % 64 || d->hidden > 8192 || d->inter > 16384) return FLINT_UNSUPPORTED;
    if ((int64_t)T * (d->hidden > d->inter ? d->hidden : d->inter) >= (int64_t)1 << 40) return FLINT_UNSUPPORTED;
    return FLINT_OK;
}

// A dense layer runs on the expert kernels as a layer with no routed experts
// (K = 0, I = 0) whose shared expert has the dense width.  Its down product has
// few column tiles per row tile (H/64 on the 32-row tiles, H/32 on the
// streaming kernels), so the reduction is split into `dense_splits` partial
// arrays that the combine adds.
int dense_splits(const flint_dense_dims *d, int32_t T)
{
    if (expert_tiles_for(T, d->hidden, 1, 0, 0, d->inter, d->dtype == FLINT_BF16).tiled)
        return tiled_dense_splits(T, d->hidden, d->inter);
    if (T > kStreamMaxT || !stream_eligible(T, d->hidden, 0, d->inter)) return 1;
    int best = 1;
    for (int s = 2; s <= 8; ++s)  // whole, even batches of 32-wide slices per wave in every split
        if (d->inter % s == 0 && stream_eligible(T, d->hidden, 0, d->inter / s)) best = s;
    return best;
}

Workspace dense_workspace(const flint_dense_dims *d, int32_t T, void *base, const void *out = nullptr)
{
    return plan_workspace_out(base, out, T, d->hidden, 1, 0, 0, d->inter, d->dtype == FLINT_BF16 ? 2 : 4,
                              dense_splits(d, T));
}

}  // namespace

extern "C" {

size_t flint_dense_workspace_bytes(const flint_dense_dims *d, int32_t T)
{
    if (check_dense(d, T) != FLINT_OK) return 0;
    return dense_workspace(d, T, nullptr).bytes;
}

flint_status flint_dense_mlp(const flint_dense_dims *d, int32_t T, const void *x, const void *gate,
                             const void *up, const void *down, void *out, flint_dtype out_dtype, void *ws,
                             size_t ws_bytes, void *stream, void *const *events)
{
    flint_status st = check_dense(d, T);
    if (st != FLINT_OK) return st;
    if (out_dtype != FLINT_F32 && out_dtype != FLINT_BF16) return FLINT_UNSUPPORTED;
    if (T == 0) return FLINT_OK;
    if (!x || !gate || !up || !down || !out) return FLINT_INVALID_ARG;
    if (!aligned16(x) || !aligned16(gate) || !aligned16(up) || !aligned16(down) || !aligned16(out))
        return FLINT_UNSUPPORTED;
    if (ws_bytes < flint_dense_workspace_bytes(d, T)) return FLINT_WORKSPACE_TOO_SMALL;
    if (!ws) return FLINT_INVALID_ARG;
    if (((uintptr_t)ws & (kAlign - 1)) != 0) return FLINT_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = d->dtype == FLINT_BF16;
    Workspace w = dense_workspace(d, T, ws, out);
    ExpertArgs e{};
    e.bf16 = bf16;
    e.T = T;
    e.H = d->hidden;
    e.E = 1;
    e.K = 0;
    e.I = 0;
    e.Is = d->inter;
    e.x = x;
    e.shared_gate = gate;
    e.shared_up = up;
    e.shared_down = down;
    e.offsets = w.offsets;
    e.list1 = w.list1;
    e.list2 = w.list2;
    e.meta = w.meta;
    e.h_sorted = w.h_sorted;
    e.h_shared = w.h_shared;
    e.y_sorted = w.y_sorted;
    e.out = out;
    e.out_bf16 = out_dtype == FLINT_BF16;
    e.shared_splits = dense_splits(d, T);
    // float32 output from a single down product: the down stage writes it directly
    e.skip_combine = out_dtype == FLINT_F32 && e.shared_splits == 1;
    e.y_shared = e.skip_combine ? (float *)out : w.y_shared;
    e.tiles = expert_tiles_for(T, d->hidden, 1, 0, 0, d->inter, bf16);
    e.cus = device_cus();
    Marks marks[3];
    if (events)
        for (int i = 0; i < 3; ++i) marks[i] = Marks{(hipEvent_t)events[2 * i], (hipEvent_t)events[2 * i + 1]};
    if (launch_experts(e, s, events ? marks : nullptr) != hipSuccess) return FLINT_DEVICE_ERROR;
    if (events && e.skip_combine) {
        if (hipEventRecord(marks[2].start, s) != hipSuccess || hipEventRecord(marks[2].stop, s) != hipSuccess)
            return FLINT_DEVICE_ERROR;
    }
    return FLINT_OK;
}

flint_status flint_rmsnorm(int32_t T, int32_t H, const float *in, void *out_bf16, float eps, void *stream)
{
    if (T < 0 || H <= 0) return FLINT_INVALID_ARG;
    if (H % 64 || H > 8192) return FLINT_UNSUPPORTED;
    if (T == 0) return FLINT_OK;
    if (!in || !out_bf16) return FLINT_INVALID_ARG;
    if (!aligned16(in) || !aligned16(out_bf16)) return FLINT_UNSUPPORTED;
    if (!(eps >= 0.0f)) return FLINT_INVALID_ARG;
    if (launch_rmsnorm(T, H, in, (uint16_t *)out_bf16, eps, (hipStream_t)stream) != hipSuccess)
        return FLINT_DEVICE_ERROR;
    return FLINT_OK;
}

}  // extern "C"
