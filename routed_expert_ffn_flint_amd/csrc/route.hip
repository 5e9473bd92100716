// Router and dispatch kernels for the Flint MoE layer (gfx950).
//
// Router: serving-kit review, "The architecture, from the config" -- sigmoid
// router scores with normalised top-k (not softmax); 256 experts, 6 per token.
// Dispatch: release news page, "What runs on each token" -- each token goes to
// the experts the router picked; grouping the (token, expert) pairs by expert
// turns the per-expert work into dense row blocks.
//
//   k_router_logits  z[t][e] = x[t] . router[e] (+ bias[e])   MFMA, fp32 accumulate
//                    (batches below 1024 tokens; larger ones use the tiled GEMM)
//   k_topk_wave      one token per wave (up to 4096 tokens): fp32 sigmoid
//                    scores, the K-th largest found by a bitwise search with
//                    wave-wide counts, ties to the lower expert index, weights
//                    s / sum(s) over the K selected
//   k_topk<16>       the same selection, 16 lanes per token, by merging sorted
//                    candidate lists (larger batches)
//   k_dispatch_tile  per tile of 256 tokens: a per-expert bitmask of the tile's
//                    tokens gives each pair its rank among earlier tokens of
//                    the tile and the tile's per-expert histogram.  When the
//                    whole batch is one tile the same work-group also scans the
//                    counts, scatters the permutation and writes the expert
//                    kernels' tile lists.
//   k_topk_dispatch_small  up to 16 tokens: the top-k of k_topk_wave and the
//                    one-tile dispatch in a single work-group
//   k_topk_dispatch_last  17 to 128 tokens in a layer call: the top-k of
//                    k_topk_wave, and the one-tile dispatch in the work-group
//                    that finishes last
//   k_dispatch_scan  (more than one tile) column scan of the tile histograms,
//                    expert offsets, tile lists (in a layer call the last
//                    k_dispatch_tile work-group does this instead).
//   k_dispatch_scatter (more than one tile) slot = offset + tile base + rank.
#include <climits>

constexpr int kTopkWaveT = 4096;  // largest batch selected one token per wave (16 lanes per token above)
// Largest batch whose top-k and dispatch run as one work-group of 16 waves,
// one token per wave (T = 8: 10.2 -> 7.4 us; with two tokens per wave their
// latencies add up: T = 32 9.8 -> 12.9 us).
constexpr int kTopkFusedT = 16;
// Largest batch of a layer call whose top-k and dispatch run as one launch of
// many work-groups, the dispatch in the last one (k_topk_dispatch_last; top-k
// + dispatch T = 32 10.0 -> 8.3 us, T = 128 10.5 -> 9.5; at T = 256 one
// work-group of 256 threads dispatching 1536 pairs was slower than the
// 1024-thread dispatch kernel, 12.5 -> 12.9 us).
constexpr int kTopkLastMaxT = 128;

#include "gemm_core.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace flint {

// ---------------------------------------------------------------------------
// Router logits.  SPLIT > 1: SPLIT waves compute the same 16x16 tile over
// slices of H and add their partial sums in wave order (many small
// work-groups, each wave one batch of loads: the decode case, where the
// latency of reading the 1 MiB router matrix matters more than reuse).
// SPLIT == 1: 4 waves in a 2x2 grid, each (MB*16) tokens x (NB*16) experts
// over all of H.
// zero / nzero: words to set to 0 besides (the fused decode kernel's counters).
template <typename DT, int MB, int NB, int SPLIT>
__global__ __launch_bounds__(SPLIT > 1 ? SPLIT * 64 : 256) void k_router_logits(
    const typename DT::storage *__restrict__ x, int T, int H, const typename DT::storage *__restrict__ router,
    const float *__restrict__ bias, int E, float *__restrict__ z, int32_t *__restrict__ zero, int nzero)
{
    if (zero) {
        const int nthreads = gridDim.x * gridDim.y * gridDim.z * blockDim.x;
        const int id = ((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
        for (int i = id; i < nzero; i += nthreads) zero[i] = 0;
    }
    using S = typename DT::storage;
    constexpr bool SPLITK = SPLIT > 1;
    constexpr int WM = SPLITK ? 1 : 2, WN = SPLITK ? 1 : 2;
    constexpr int TILE_T = WM * MB * 16, TILE_E = WN * NB * 16;
    __shared__ float red[SPLITK ? SPLIT * MB * NB * 256 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = SPLITK ? 0 : wave / WN, wn = SPLITK ? 0 : wave % WN;
    const int t0 = blockIdx.y * TILE_T + wm * MB * 16;
    const int e0 = blockIdx.x * TILE_E + wn * NB * 16;
    // blockIdx.z: which of gridDim.z slices of H this work-group sums (its
    // own partial array; the bias goes into the first)
    const int hz = H / gridDim.z, kz = blockIdx.z * hz;
    const int kg = kz + (lane >> 4) * 8;
    z += (size_t)blockIdx.z * T * E;
    if (blockIdx.z != 0) bias = nullptr;

    const S *a_rows[MB];
    const S *b_rows[NB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        int t = t0 + m * 16 + (lane & 15);
        if (t >= T) t = blockIdx.y * TILE_T;  // inside the tile's first row: valid, result dropped
        a_rows[m] = x + (size_t)t * H + kg;
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        int e = e0 + n * 16 + (lane & 15);
        if (e >= E) e = 0;
        b_rows[n] = router + (size_t)e * H + kg;
    }

    f32x4 acc[MB][NB];
    zero_acc(acc);
    const int nslices = hz / 32;
    int s0 = 0, s1 = nslices;
    if (SPLITK) {
        const int per = (nslices + SPLIT - 1) / SPLIT;
        s0 = min(wave * per, nslices);
        s1 = min(s0 + per, nslices);
    }
    wave_gemm<DT, MB, NB, 4>(a_rows, b_rows, s0, s1, acc);
    if (SPLITK) {
        splitk_reduce<SPLIT, MB, NB>(acc, red);
        if (wave != 0) return;
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int e = e0 + n * 16 + (lane & 15);
            if (e >= E) continue;
            const float b = bias ? bias[e] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + m * 16 + (lane >> 4) * 4 + i;
                if (t < T) z[(size_t)t * E + e] = acc[m][n][i] + b;
            }
        }
}

// Up to 128 tiles of 16 tokens x 16 experts (T = 32, E = 256: 32 tiles) each
// tile's sum over H is split between two work-groups of 8 waves, each writing
// its own partial array (top-k adds the two in order), so twice as many CUs
// read the router matrix: measured 5.8 -> 4.2 us at T = 32 and 6.1 -> 4.3 us at
// T = 128 (four or eight partial arrays cost top-k more than they save; at 256
// tiles, T = 256, the split gained nothing, 6.1 -> 6.0 us).
constexpr int kRouterSmallSplits = 2;
static_assert(kRouterSmallSplits == 1 || kRouterSmallSplits == 2 || kRouterSmallSplits == 4 ||
                  kRouterSmallSplits == 8,
              "router splits: 1, 2, 4 or 8 (16 / splits waves per work-group)");
int small_router_splits(int T, int H, int E)
{
    const long long tiles = (long long)((E + 15) / 16) * ((T + 15) / 16);
    const int s = kRouterSmallSplits;
    return s > 1 && tiles <= 128 && H % (32 * s) == 0 ? s : 1;
}

hipError_t launch_router_logits(bool bf16, const void *x, int T, int H, const void *router,
                                const float *bias, int E, float *logits, hipStream_t stream, Marks m,
                                int32_t *zero, int nzero)
{
    if (T <= 0) return hipSuccess;
    if (tiled_router_eligible(T, H, bf16)) {
        if (zero) return hipErrorInvalidValue;  // (the counters belong to batches below 1024 tokens)
        return launch_router_tiled(x, T, H, router, bias, E, logits, stream, m);
    }
    const uint16_t *xb = (const uint16_t *)x, *rb = (const uint16_t *)router;
    const float *xf = (const float *)x, *rf = (const float *)router;
    if (T < 1024) {
        // 16 waves per 16x16 tile, each wave 1/16 of H (at H = 2048: four
        // 32-wide slices), in small_router_splits(H) work-groups of 16 / that
        // many waves, each writing its own partial array
        const int zs = small_router_splits(T, H, E);
        dim3 grid((E + 15) / 16, (T + 15) / 16, zs);
        const int thr = 1024 / zs;
#define FLINT_ROUTER_LAUNCH(W)                                                                              \
    return bf16 ? launch_k(k_router_logits<BF16, 1, 1, W>, grid, thr, 0, stream, m, xb, T, H, rb, bias, E, logits, \
                           zero, nzero)                                                                        \
                : launch_k(k_router_logits<F32, 1, 1, W>, grid, thr, 0, stream, m, xf, T, H, rf, bias, E, logits, \
                           zero, nzero)
        switch (zs) {
        case 2: FLINT_ROUTER_LAUNCH(8);
        case 4: FLINT_ROUTER_LAUNCH(4);
        case 8: FLINT_ROUTER_LAUNCH(2);
        default: FLINT_ROUTER_LAUNCH(16);
        }
#undef FLINT_ROUTER_LAUNCH
    }
    dim3 grid((E + 127) / 128, (T + 63) / 64);
    if (bf16)
        return launch_k(k_router_logits<BF16, 2, 4, 1>, grid, 256, 0, stream, m, xb, T, H, rb, bias, E, logits, zero,
                        nzero);
    return launch_k(k_router_logits<F32, 2, 4, 1>, grid, 256, 0, stream, m, xf, T, H, rf, bias, E, logits, zero,
                    nzero);
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scans of three ints per thread over the first 256
// threads (threads beyond 256 contribute 0), with two barriers for all three.
// Every thread of the block must call it; lds holds 12 ints.
__device__ void block_exclusive_scan256x3(const int (&v)[3], int *lds, int (&excl)[3], int (&total)[3])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) incl[j] = threadIdx.x < 256 ? v[j] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int y = __shfl_up(incl[j], off, 64);
            if (lane >= off) incl[j] += y;
        }
    if (lane == 63 && wave < 4)
#pragma unroll
        for (int j = 0; j < 3; ++j) lds[4 * j + wave] = incl[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        int base = 0;
        for (int w = 0; w < 4 && w < wave; ++w) base += lds[4 * j + w];
        total[j] = lds[4 * j] + lds[4 * j + 1] + lds[4 * j + 2] + lds[4 * j + 3];
        excl[j] = base + incl[j] - (threadIdx.x < 256 ? v[j] : 0);
    }
    __syncthreads();
}

// Counts -> offsets and the expert kernels' tile lists.  Thread e < E holds
// counts[e] in `c`.  lists: entry i = (expert, first slot of the tile).
__device__ int finish_offsets_and_lists(int c, int E, int32_t *offsets, int32_t *counts,
                                        int32_t *list1, int bm1, int32_t *list2, int bm2,
                                        int32_t *meta, int *lds)
{
    const int e = threadIdx.x;
    const bool own = e < E;
    if (!own) c = 0;
    // slots, gate/up tiles and down tiles of each expert
    const int n[3] = {c, (c + bm1 - 1) / bm1, (c + bm2 - 1) / bm2};
    int ex[3], tot[3];
    block_exclusive_scan256x3(n, lds, ex, tot);
    const int off = ex[0], total = tot[0], n1 = n[1], n2 = n[2], st1 = ex[1], st2 = ex[2];
    const int tot1 = tot[1], tot2 = tot[2];
    if (own) {
        counts[e] = c;
        offsets[e] = off;
        if (e == E - 1) offsets[E] = total;
        for (int i = 0; i < n1; ++i) {
            list1[2 * (st1 + i)] = e;
            list1[2 * (st1 + i) + 1] = off + i * bm1;
        }
        for (int i = 0; i < n2; ++i) {
            list2[2 * (st2 + i)] = e;
            list2[2 * (st2 + i) + 1] = off + i * bm2;
        }
    }
    if (threadIdx.x == 0) {
        meta[0] = tot1;
        meta[1] = tot2;
    }
    return off;  // expert threadIdx.x's first slot
}

// Selection key of a candidate: larger key = selected first.  Scores are
// sigmoids (>= 0), whose float32 bit patterns order like the values, so the key
// orders by score and then, for equal scores, by lower expert index.  Key 0 is
// below every real candidate (used for experts past E and for padding).
__device__ __forceinline__ uint64_t sel_key(float s, int e)
{
    return ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return (int)(0xffffffffu - (uint32_t)k); }
__device__ __forceinline__ float key_score(uint64_t k) { return __uint_as_float((uint32_t)(k >> 32)); }

__device__ __forceinline__ void cas_desc(uint64_t &a, uint64_t &b)
{
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = hi;
    b = lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off)
{
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    return ((uint64_t)(uint32_t)__shfl_xor((int)hi, off, 64) << 32) | (uint32_t)__shfl_xor((int)lo, off, 64);
}

// Top-8 keys (descending) of one token, computed by a group of G lanes (G = 16
// or 64): each lane sorts its 256/G candidates (experts gl + G*i) into a list
// of the best 8, then log2(G) butterfly steps merge the lists across the group
// -- the better half of two sorted lists is the element-wise larger of one list
// and the other reversed (a bitonic sequence), which a 3-stage bitonic network
// sorts.  Every lane of the group ends with the same list.
template <int G>
__device__ __forceinline__ void group_top8(const float *zt, size_t split_stride, int nsplit, int E,
                                           uint64_t (&l)[kMaxTopK])
{
    constexpr int C = kMaxExperts / G;
    const int gl = threadIdx.x & (G - 1);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) l[j] = 0;
    // every load unconditional (experts past E read expert 0 and are masked),
    // so they go out together instead of one latency each
    float zs[C];
#pragma unroll
    for (int i = 0; i < C; ++i) zs[i] = zt[gl + G * i < E ? gl + G * i : 0];
    for (int sp = 1; sp < nsplit; ++sp)  // partial sums, in order
#pragma unroll
        for (int i = 0; i < C; ++i) zs[i] += zt[sp * split_stride + (gl + G * i < E ? gl + G * i : 0)];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int e = gl + G * i;
        uint64_t k = e < E ? sel_key(score_from_logit(zs[i]), e) : 0;
        if (C <= kMaxTopK) {
            l[i] = k;  // fewer candidates than list slots: keep all, sort below
        } else if (k > l[kMaxTopK - 1]) {
            l[kMaxTopK - 1] = k;
#pragma unroll
            for (int j = kMaxTopK - 1; j > 0; --j) cas_desc(l[j - 1], l[j]);
        }
    }
    if (C <= kMaxTopK) {
        // sort the C (<= 8) kept keys; padding keys are 0
#pragma unroll
        for (int i = 1; i < kMaxTopK; ++i)
#pragma unroll
            for (int j = i; j > 0; --j) cas_desc(l[j - 1], l[j]);
    }
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
        uint64_t p[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) p[j] = shfl_xor_u64(l[j], off);
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) l[j] = l[j] > p[kMaxTopK - 1 - j] ? l[j] : p[kMaxTopK - 1 - j];
#pragma unroll
        for (int half = kMaxTopK / 2; half >= 1; half >>= 1)
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if ((j & half) == 0) cas_desc(l[j], l[j + half]);
    }
}

// Top-k for every token: groups of G lanes, one token per group, many
// work-groups (the selection is arithmetic-heavy, so it is spread over the
// whole chip).  Writes topk_idx (ascending expert ids) and topk_w.
// LDS of one tile's dispatch.
struct TileLds {
    int16_t sel[kTopkTile * kMaxTopK];
    uint32_t masks[kMaxExperts * (kTopkTile / 32)];
    int32_t offs[kMaxExperts];
    int lds[12];
};

// Dispatch of one tile of up to 256 tokens by a work-group of NT threads: a
// per-expert bitmask of the tile's tokens gives each (token, expert) pair its
// rank among earlier tokens of the tile (a popcount of the lower bits), and
// the tile's per-expert histogram.  When the whole batch is one tile
// (`single`) the same work-group also scans the counts, scatters the
// permutation and writes the expert kernels' tile lists.
// coherent: read the selection with agent-coherent loads (other work-groups of
// the same launch wrote it).
template <int NT>
__device__ void dispatch_tile(const DispatchArgs &a, int tile, bool single, TileLds &L, bool sel_in_lds,
                              bool coherent = false)
{
    constexpr int PER = kTopkTile * kMaxTopK / NT;  // pairs per thread, at most
    constexpr int W = kTopkTile / 32;
    const int E = a.E, K = a.K;
    const int t_base = tile * kTopkTile;
    const int tile_len = min(kTopkTile, a.T - t_base);

    if (!sel_in_lds)
        for (int i = threadIdx.x; i < tile_len * K; i += NT) {
            const int32_t *p = a.topk_idx + (size_t)t_base * K + i;
            L.sel[i] = (int16_t)(coherent ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p);
        }
    for (int i = threadIdx.x; i < E * W; i += NT) L.masks[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < tile_len * K; i += NT) {
        const int tl = i / K, e = L.sel[i];
        atomicOr(&L.masks[e * W + (tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    int my_rank[PER];
    int my_e[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int i = threadIdx.x + r * NT;
        my_e[r] = -1;
        my_rank[r] = 0;
        if (i < tile_len * K) {
            const int tl = i / K, e = L.sel[i];
            int rk = __popc(L.masks[e * W + (tl >> 5)] & ((1u << (tl & 31)) - 1u));
            for (int w = 0; w < (tl >> 5); ++w) rk += __popc(L.masks[e * W + w]);
            my_rank[r] = rk;
            my_e[r] = e;
        }
    }
    int hcount = 0;
    if (threadIdx.x < E)
        for (int w = 0; w < W; ++w) hcount += __popc(L.masks[threadIdx.x * W + w]);

    if (!single) {
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int i = threadIdx.x + r * NT;
            if (my_e[r] >= 0) a.rank[(size_t)t_base * K + i] = my_rank[r];
        }
        if (threadIdx.x < E) {
            int32_t *h = a.hist + (size_t)tile * E + threadIdx.x;
            if (a.done)  // the last tile's work-group reads it in this launch
                __hip_atomic_store(h, hcount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                *h = hcount;
        }
        return;
    }
    const int off = finish_offsets_and_lists(hcount, E, a.offsets, a.counts, a.list1, a.bm1, a.list2, a.bm2,
                                             a.meta, L.lds);
    if (a.y_scale) {
        // the fp16 output exponents start at 0 (for several tiles the scatter
        // kernel clears them): the T*K routed rows and the T shared rows
        // (16 bytes a store: the workspace's arrays start 256-byte aligned)
        const int n = (a.T * K + a.T) * a.scale_cols;
        uint4 *y16 = reinterpret_cast<uint4 *>(a.y_scale);
        for (int i = threadIdx.x; i < n / 16; i += NT) y16[i] = make_uint4(0u, 0u, 0u, 0u);
        for (int i = n / 16 * 16 + threadIdx.x; i < n; i += NT) a.y_scale[i] = 0;
    }
    if (threadIdx.x < E) L.offs[threadIdx.x] = off;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int i = threadIdx.x + r * NT;
        if (my_e[r] >= 0) {
            const int slot = L.offs[my_e[r]] + my_rank[r];
            a.sorted_token[slot] = t_base + i / K;
            a.slot_of[(size_t)t_base * K + i] = slot;
        }
    }
}

// The K best keys of a token, written in ascending expert order with weights
// s / sum(s) (the sum taken in double in that order); lane gl writes entry gl.
__device__ __forceinline__ void write_topk(const uint64_t (&l)[kMaxTopK], int t, int K, int gl,
                                           int32_t *__restrict__ topk_idx, float *__restrict__ topk_w)
{
    // the K best, in ascending expert order
    int se[kMaxTopK];
    float ss[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        se[k] = k < K ? key_expert(l[k]) : INT_MAX;
        ss[k] = key_score(l[k]);
    }
#pragma unroll
    for (int i = 1; i < kMaxTopK; ++i)
#pragma unroll
        for (int j = i; j > 0; --j)
            if (se[j] < se[j - 1]) {
                const int te = se[j];
                se[j] = se[j - 1];
                se[j - 1] = te;
                const float ts = ss[j];
                ss[j] = ss[j - 1];
                ss[j - 1] = ts;
            }
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K) sum += (double)ss[k];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K && gl == k) {
            topk_idx[(size_t)t * K + k] = se[k];
            topk_w[(size_t)t * K + k] = routing_weight(ss[k], sum, K);
        }
}

// Top-K of one token by one wave (wave_topk_select), written out: topk_idx
// (ascending ids) and topk_w, and for a one-tile batch the selection in LDS.
__device__ __forceinline__ void wave_topk(const float *zt, size_t split_stride, int nsplit, int E, int K, int t,
                                          int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
                                          float *ls, int *le, int16_t *sel_lds = nullptr)
{
    const int lane = threadIdx.x & 63;
    int idx;
    float w;
    wave_topk_select(zt, split_stride, nsplit, E, K, ls, le, idx, w);
    if (lane < K) {
        topk_idx[(size_t)t * K + lane] = idx;
        topk_w[(size_t)t * K + lane] = w;
        if (sel_lds) sel_lds[t * K + lane] = (int16_t)idx;  // (a one-tile batch: t is tile-relative)
    }
}

__global__ __launch_bounds__(256) void k_topk_wave(DispatchArgs da)
{
    __shared__ float ls[4][kMaxTopK];
    __shared__ int le[4][kMaxTopK];
    const int wave = threadIdx.x >> 6;
    const int tok = blockIdx.x * 4 + wave;
    if (da.done && da.dispatch && da.T > kTopkTile && blockIdx.x == 0 && threadIdx.x == 0)
        *da.done = 0;  // for the dispatch kernels that follow (several tiles)
    if (tok >= da.T) return;  // whole waves
    wave_topk(da.logits + (size_t)tok * da.E, (size_t)da.T * da.E, da.logit_splits, da.E, da.K, tok, da.topk_idx,
              da.topk_w, ls[wave], le[wave]);
}

template <int G>
__global__ __launch_bounds__(256) void k_topk(DispatchArgs da)
{
    const float *__restrict__ logits = da.logits;
    const int T = da.T, E = da.E, K = da.K;
    int32_t *__restrict__ topk_idx = da.topk_idx;
    float *__restrict__ topk_w = da.topk_w;
    const int groups_per_block = blockDim.x / G;
    const int tok = blockIdx.x * groups_per_block + threadIdx.x / G;
    const int gl = threadIdx.x & (G - 1);
    const int t = tok < T ? tok : T - 1;  // whole groups share a token; extra groups redo the last one
    if (da.done && da.dispatch && T > kTopkTile && blockIdx.x == 0 && threadIdx.x == 0)
        *da.done = 0;  // for the dispatch kernels that follow (several tiles)
    uint64_t l[kMaxTopK];
    group_top8<G>(logits + (size_t)t * E, (size_t)T * E, da.logit_splits, E, l);
    if (tok < T) write_topk(l, t, K, gl, topk_idx, topk_w);
}

__device__ void scan_tiles(const DispatchArgs &a, int ntiles, int *lds, bool coherent);

// Several tiles with a.done: the work-group that finishes its tile last (its
// histogram stores acknowledged first, like every other's) also scans the
// histograms, in place of k_dispatch_scan.
__global__ __launch_bounds__(1024) void k_dispatch_tile(DispatchArgs a, int fused_single_tile)
{
    __shared__ TileLds L;
    __shared__ int is_last;
    dispatch_tile<1024>(a, blockIdx.x, fused_single_tile != 0, L, false);
    if (fused_single_tile || !a.done) return;
    wait_vmcnt<0>();  // this wave's histogram stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
    __syncthreads();
    if (!is_last) return;
    scan_tiles(a, gridDim.x, L.lds, true);
}

// Small batches (up to 16 tokens): top-k (one token per wave, 16 waves) and
// the whole dispatch in one work-group; the selection reaches the dispatch
// through LDS.  One launch instead of two, and no round trip of topk_idx
// through memory.
__global__ __launch_bounds__(1024) void k_topk_dispatch_small(DispatchArgs a)
{
    __shared__ TileLds L;
    __shared__ float ls[16][kMaxTopK];
    __shared__ int le[16][kMaxTopK];
    const int wave = threadIdx.x >> 6;
    for (int t = wave; t < a.T; t += 16)
        wave_topk(a.logits + (size_t)t * a.E, (size_t)a.T * a.E, a.logit_splits, a.E, a.K, t, a.topk_idx, a.topk_w,
                  ls[wave], le[wave], L.sel);
    __syncthreads();
    dispatch_tile<1024>(a, 0, true, L, true);
}

// 17 to kTopkLastMaxT tokens (one tile): the top-k of k_topk_wave (one token
// per wave, four per work-group), and the dispatch in the work-group that
// finishes its tokens last, counted on a.done (zeroed by the router kernel
// before): one launch instead of two.  The selection crosses work-groups through
// agent-coherent stores, acknowledged (vmcnt 0) before the counter is raised,
// and agent-coherent loads in the last work-group; no work-group waits for
// another.
__global__ __launch_bounds__(256) void k_topk_dispatch_last(DispatchArgs a)
{
    __shared__ TileLds L;
    __shared__ float ls[4][kMaxTopK];
    __shared__ int le[4][kMaxTopK];
    __shared__ int is_last;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t < a.T) {
        int idx;
        float w;
        wave_topk_select(a.logits + (size_t)t * a.E, (size_t)a.T * a.E, a.logit_splits, a.E, a.K, ls[wave],
                         le[wave], idx, w);
        if (lane < a.K) {
            __hip_atomic_store(a.topk_idx + (size_t)t * a.K + lane, idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            a.topk_w[(size_t)t * a.K + lane] = w;
        }
    }
    wait_vmcnt<0>();  // this wave's stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
    __syncthreads();
    if (!is_last) return;
    dispatch_tile<256>(a, 0, true, L, false, true);
}

// More than one tile: per-expert column scan of the tile histograms.
// Thread e < E scans expert e's column of the tile histograms (coherent: with
// agent-coherent loads, the histograms written by other work-groups of the
// same launch); then the offsets and the tile lists.  Every thread of the
// work-group (at least 256) calls it; lds holds 12 ints.
__device__ void scan_tiles(const DispatchArgs &a, int ntiles, int *lds, bool coherent)
{
    const int e = threadIdx.x;
    int run = 0;
    if (e < a.E) {
        for (int tile = 0; tile < ntiles; tile += 8) {
            int h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t *p = a.hist + (size_t)(tile + j < ntiles ? tile + j : 0) * a.E + e;
                const int v = coherent ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
                h[j] = tile + j < ntiles ? v : 0;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (tile + j < ntiles) a.tile_base[(size_t)(tile + j) * a.E + e] = run;
                run += h[j];
            }
        }
    }
    finish_offsets_and_lists(run, a.E, a.offsets, a.counts, a.list1, a.bm1, a.list2, a.bm2,
                             a.meta, lds);
}

__global__ __launch_bounds__(256) void k_dispatch_scan(DispatchArgs a, int ntiles)
{
    __shared__ int lds[12];
    scan_tiles(a, ntiles, lds, false);
}

__global__ __launch_bounds__(256) void k_dispatch_scatter(DispatchArgs a)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.T * a.K) return;
    if (a.y_scale) {  // the fp16 output exponents start at 0
        for (int c = 0; c < a.scale_cols; ++c) a.y_scale[(size_t)i * a.scale_cols + c] = 0;
        if (i < a.T)  // the shared expert's rows follow the T*K routed ones
            for (int c = 0; c < a.scale_cols; ++c) a.y_scale[((size_t)a.T * a.K + i) * a.scale_cols + c] = 0;
    }
    const int t = i / a.K;
    const int e = a.topk_idx[i];
    const int tile = t / kTopkTile;
    const int slot = a.offsets[e] + a.tile_base[(size_t)tile * a.E + e] + a.rank[i];
    a.sorted_token[slot] = t;
    a.slot_of[i] = slot;
}

__global__ void k_fill_i32(int32_t *p, int n, int32_t value)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t value, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    k_fill_i32<<<(n + 255) / 256, 256, 0, stream>>>(p, n, value);
    return hipGetLastError();
}

hipError_t launch_topk_dispatch(const DispatchArgs &a, hipStream_t stream, Marks m)
{
    if (a.T <= 0) return hipSuccess;
    const int ntiles = (a.T + kTopkTile - 1) / kTopkTile;
    const int fused = (ntiles == 1) ? 1 : 0;
    // the first kernel carries m.start, the last m.stop
    Marks first{m.start, a.dispatch ? nullptr : m.stop};
    hipError_t err = hipSuccess;
    if (a.compute_topk && a.dispatch && fused && a.T <= kTopkFusedT && a.E <= 256)
        return launch_k(k_topk_dispatch_small, 1, 1024, 0, stream, m, a);
    if (a.compute_topk && a.dispatch && fused && a.done && a.T <= kTopkLastMaxT && a.E <= 256)
        return launch_k(k_topk_dispatch_last, (a.T + 3) / 4, 256, 0, stream, m, a);
    if (a.compute_topk) {
        err = a.T <= kTopkWaveT ? launch_k(k_topk_wave, (a.T + 3) / 4, 256, 0, stream, first, a)
                          : launch_k(k_topk<16>, (a.T + 15) / 16, 256, 0, stream, first, a);
        if (err != hipSuccess) return err;
        first.start = nullptr;
    }
    if (a.dispatch) {
        // several tiles: the last tile work-group scans the histograms when the
        // top-k kernel above has cleared the counter; else k_dispatch_scan does
        DispatchArgs b = a;
        if (!a.compute_topk) b.done = nullptr;
        err = launch_k(k_dispatch_tile, ntiles, 1024, 0, stream, Marks{first.start, fused ? m.stop : nullptr}, b,
                       fused);
        if (err != hipSuccess || fused) return err;
        if (!b.done) {
            err = launch_k(k_dispatch_scan, 1, 256, 0, stream, Marks{}, b, ntiles);
            if (err != hipSuccess) return err;
        }
        err = launch_k(k_dispatch_scatter, (a.T * a.K + 255) / 256, 256, 0, stream, Marks{nullptr, m.stop}, b);
    }
    return err;
}

}  // namespace flint
