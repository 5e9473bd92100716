// Host-side launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace flint {

// Timing marks of one stage (either may be null).  A kernel launched through
// launch_k with a non-null mark has it stamped by the runtime when that kernel
// itself begins (start) or ends (stop), so a stage's interval is its kernels'
// execution time, without the queue gaps around them.
struct Marks {
    hipEvent_t start = nullptr, stop = nullptr;
};

// kernel<<<grid, block, lds, s>>>(args...), through hipExtLaunchKernel when a
// mark is given.  Returns hipGetLastError() / the launch status.
template <typename... P, typename... A>
hipError_t launch_k(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, Marks m, A &&...args)
{
    if (!m.start && !m.stop) {
        kernel<<<grid, block, lds, s>>>(std::forward<A>(args)...);
        return hipGetLastError();
    }
    std::tuple<P...> vals{std::forward<A>(args)...};
    void *ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1];
    std::apply(
        [&ptrs](auto &...v) {
            int i = 0;
            ((ptrs[i++] = (void *)&v), ...);
        },
        vals);
    return hipExtLaunchKernel((const void *)kernel, grid, block, ptrs, lds, s, m.start, m.stop, 0);
}

// Tokens per work-group in the top-k / dispatch kernels.
constexpr int kTopkTile = 256;
// Maximum supported sizes.
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;
// Largest batch the persistent weight-streaming expert kernels (and the
// split-k small-batch kernels) serve.
constexpr int kStreamMaxT = 512;
// Where the LDS-tiled kernels take over when the shape allows them (bf16).
// A MoE layer: from 160 rows on 16-row tiles (Flint shape, layer time against
// the weight-streaming kernels: T = 192 328 -> 313 us, 256 338 -> 318, 384
// 376 -> 346; even at 128, slower at 64), from 513 rows on the 128- and
// 256-row tiles (T = 640: 398 -> 373 us; at 448 and 512 the 16-row tiles are
// 1-2% faster).  A dense layer at every T: 32-row tiles below 129 rows, the
// large tiles from there (its weights the streaming kernels read again for
// every 32 rows).
constexpr int kTiledFromT = 160;
constexpr int kLargeTilesFromT = 513;
constexpr int kDenseTiledFromT = 129;

// The persistent fused decode kernel (fused.hip): queues (work-group classes),
// largest batch, most shared-expert slices, and its counter words.
constexpr int kFusedQueues = 8;
constexpr int kFusedMaxT = 64;
constexpr int kFusedMaxShared = 8;
constexpr int kFusedSyncWords = (2 * kFusedQueues + kMaxExperts + kFusedMaxShared + 1) * 32;

// Columns that share one exponent of the fp16 routed outputs (y16).
constexpr int kYScaleCols = 64;

// Tile shapes of the expert kernels for one launch regime.
struct ExpertTiles {
    int bm1;  // rows per gate/up tile
    int bn1;  // intermediate channels per gate/up tile
    int bm2;  // rows per down tile
    int bn2;  // output columns per down tile
    bool small;   // split-k decode kernels (true) or tiled kernels (false)
    bool stream;  // small batches on the persistent weight-streaming kernels
    bool tiled;   // large bf16 batches on the LDS-tiled kernels
};

// Tile shapes (and with them the dispatch's tile lists) for T tokens of a
// layer with these sizes.
ExpertTiles expert_tiles_for(int T, int H, int E, int K, int I, int Is, bool bf16);

// Device pointers carved out of the caller's workspace.
struct Workspace {
    float *logits;        // [splits][T][E] (partial sums over slices of H; see router_splits)
    int32_t *hist;        // [ntiles][E]
    int32_t *tile_base;   // [ntiles][E]
    int32_t *rank;        // [T*K]
    int32_t *topk_idx;    // [T*K] (used when the caller passes none)
    float *topk_w;        // [T*K]
    int32_t *counts;      // [E]
    int32_t *offsets;     // [E+1]
    int32_t *sorted_token;  // [T*K]
    int32_t *slot_of;     // [T*K]
    int32_t *list1;       // [2*cap1] gate/up tile list (expert, first slot)
    int32_t *list2;       // [2*cap2] down tile list
    int32_t *meta;        // [4]: list1 length, list2 length
    void *h_sorted;       // [T*K][I] dtype
    void *h_shared;       // [T][Is] dtype
    float *y_sorted;      // [T*K][H] float32, or fp16 (with y_scale) on the tiled kernels
    float *y_shared;      // [T][H]
    int8_t *y_scale;      // [T*K + T][H/64]: power-of-two exponents of fp16 y_sorted, then of fp16 y_shared
    int32_t *topk_q;      // fused decode: [queues][T][K] per-queue copies of the selection
    int32_t *sync;        // fused decode: kFusedSyncWords counters
    int32_t *done;        // [1] top-k / dispatch work-groups finished (DispatchArgs::done)
    size_t bytes;         // total bytes needed
};

// Computes the layout for (T, dims); with base == nullptr only .bytes is valid.
// shared_splits: partial arrays of the shared expert's down product (y_shared
// is [shared_splits][T][H]; see ExpertArgs::shared_splits).
Workspace plan_workspace(void *base, int T, int H, int E, int K, int I, int Is, int elem_bytes,
                         int shared_splits = 1);

int list_capacity(int T, int K, int E, int bm);

// Compute units of the current device (read once per device).
int device_cus();

// ---- launches (all enqueue on `stream`, return hipGetLastError()) ----------

// Number of partial logit arrays the router writes (the sum over slices of H
// is split for batches of 1024-4096 tokens, and below 1024 when the batch has
// few router tiles); the top-k kernels add them in order.
int router_splits(int T, int H, int E, bool bf16);
// Partial arrays of the router product for T < 1024 (work-groups per 16x16 tile).
int small_router_splits(int T, int H, int E);

// logits[t][e] = x[t] . router[e] (+ bias[e]), float32, as router_splits
// partial arrays (bias in the first) that sum to it.
// zero / nzero: int32 words the kernel also sets to 0 (the fused decode
// kernel's counters; T < 1024 only), or null.
hipError_t launch_router_logits(bool bf16, const void *x, int T, int H, const void *router,
                                const float *bias, int E, float *logits, hipStream_t stream, Marks m = {},
                                int32_t *zero = nullptr, int nzero = 0);

// Top-k selection and/or dispatch.  See route.hip for the modes.
struct DispatchArgs {
    int T, E, K;
    const float *logits;      // when compute_topk: logit_splits arrays of [T][E] to add
    int logit_splits;
    int32_t *topk_idx;        // out when compute_topk, in otherwise
    float *topk_w;            // out when compute_topk
    bool compute_topk;
    bool dispatch;            // also produce counts/offsets/sorted_token/slot_of (+ tile lists)
    int32_t *hist, *tile_base, *rank;
    int32_t *counts, *offsets, *sorted_token, *slot_of;
    int32_t *list1, *list2, *meta;
    int bm1, bm2;
    // the exponents of the tiled down product's fp16 outputs, cleared by the
    // dispatch (its scatter kernel, or the one work-group of a single tile)
    // ([T*K + T][scale_cols] bytes: the routed rows, then the shared expert's;
    // null: none)
    int8_t *y_scale;
    int scale_cols;
    // Non-null (compute_topk and dispatch): a counter word in the workspace.
    // A one-tile batch finds it at 0 (the router kernel clears it) and, from 17
    // to 128 tokens, runs the top-k and the dispatch as one launch, the
    // dispatch in the work-group that finishes its tokens last.  With several
    // tiles the top-k kernel clears it, and the tile work-group that finishes
    // last also scans the tile histograms (no separate scan launch).
    int32_t *done;
};
hipError_t launch_topk_dispatch(const DispatchArgs &a, hipStream_t stream, Marks m = {});

struct ExpertArgs {
    bool bf16;
    bool mx4;  // expert matrices in MXFP4: gate/up/down/shared_* hold codes, *_s the scales
    int T, H, E, K, I, Is;
    const void *x;
    const void *gate, *up, *down;
    const void *shared_gate, *shared_up, *shared_down;
    const uint8_t *gate_s, *up_s, *down_s, *shared_gate_s, *shared_up_s, *shared_down_s;
    const int32_t *sorted_token, *offsets, *slot_of;
    const float *topk_w;
    const int32_t *list1, *list2, *meta;
    void *h_sorted, *h_shared;
    float *y_sorted, *y_shared;
    // The tiled down product stores routed rows of y_sorted as fp16 times
    // 2^y_scale[slot][c / 64] (an exponent per row and 64 columns, 0 unless
    // the row's 64 values reach 2^15), and the shared expert's rows of
    // y_shared likewise with exponents y_scale[T*K + t]; the combine reads
    // them back.
    bool y16;
    int8_t *y_scale;
    // The shared expert's down product split over its reduction into this many
    // partial arrays y_shared[s] (the streaming kernels only; 1 elsewhere), which
    // the combine adds in order: a dense layer at decode sizes has too few
    // column tiles to fill the chip otherwise.
    int shared_splits;
    void *out;
    bool out_bf16;
    // Non-null: the combine also writes RMSNorm of each float32 output row
    // (epsilon norm_eps) to norm_out, [T][H] bf16.
    uint16_t *norm_out;
    float norm_eps;
    bool skip_combine;  // the shared down stage writes the output itself (a dense layer, float32 out)
    ExpertTiles tiles;
    int cus;  // compute units of the device (sizes the persistent kernels' grids)
    const int32_t *fail;  // nonzero: a bounded wait of the fused decode kernel gave up (combine writes NaN)
};
// marks (nullable): 3 stages, gate/up (+ shared), down (+ shared), combine.
hipError_t launch_experts(const ExpertArgs &a, hipStream_t stream, const Marks *marks);

// Persistent streaming kernels (small batches, shapes whose H, I, Is split into
// whole batches), a few work-groups per CU.
bool stream_eligible(int T, int H, int I, int Is);
int stream_bm1(int T, int K);
int stream_bm2();
// marks (nullable): gate/up and down stages.
hipError_t launch_experts_stream(const ExpertArgs &a, hipStream_t stream, const Marks *marks);

// Streaming kernels for MXFP4 expert weights (small batches, bf16 activations):
// eligibility, rows per gate/up and per down tile (the dispatch builds its tile
// lists with these), launch of the gate/up and down stages.
constexpr int kMx4MaxT = 512;
bool mx4_eligible(int T, int H, int I, int Is);
int mx4_bm1();
int mx4_bm2();
hipError_t launch_experts_mx4(const ExpertArgs &a, hipStream_t stream, const Marks *marks);

// LDS-tiled kernels for large bf16 batches: rows per gate/up and per down tile
// (128 or 256, from the mean rows per expert), eligibility, launch.
int tiled_bm1(int T, int K, int E, int Is);
int tiled_bm2(int T, int K, int E);
bool tiled_eligible(int T, int K, int E, int H, int I, int Is, bool bf16);
hipError_t launch_experts_tiled(const ExpertArgs &a, hipStream_t stream, const Marks *marks);
// Partial arrays the down product of a dense layer (K = 0) splits its
// reduction into on the tiled kernels.
int tiled_dense_splits(int T, int H, int Is);
// The router product on the same tiles (large bf16 batches).
bool tiled_router_eligible(int T, int H, bool bf16);
constexpr int kRouterSplits = 4;
hipError_t launch_router_tiled(const void *x, int T, int H, const void *router, const float *bias, int E,
                               float *logits, hipStream_t stream, Marks m);

// The fused decode kernel (top-k, dispatch, gate/up, down in one launch) for
// bf16 batches of up to kFusedMaxT tokens: eligibility and launch.  The
// combine (launch_combine) follows it.
bool fused_eligible(int T, int H, int E, int K, int I, int Is, bool bf16);
hipError_t launch_fused_decode(const ExpertArgs &a, const float *logits, int logit_splits, int32_t *topk_idx,
                               float *topk_w, int32_t *topk_q, int32_t *sync, int32_t *counts, int32_t *offsets,
                               int32_t *sorted_token, int32_t *slot_of, hipStream_t stream, Marks m);
hipError_t launch_combine(const ExpertArgs &a, hipStream_t stream, Marks m);

hipError_t launch_fill_i32(int32_t *p, int n, int32_t value, hipStream_t stream);

hipError_t launch_rmsnorm(int T, int H, const float *in, uint16_t *out, float eps, hipStream_t stream);

}  // namespace flint
