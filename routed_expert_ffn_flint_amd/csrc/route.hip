// Router and dispatch kernels for the Flint MoE layer (gfx950).
//
// Router: serving-kit review, "The architecture, from the config" -- sigmoid
// router scores with normalised top-k (not softmax); 256 experts, 6 per token.
// Dispatch: release news page, "What runs on each token" -- each token goes to
// the experts the router picked; grouping the (token, expert) pairs by expert
// turns the per-expert work into dense row blocks.
//
//   k_router_logits  z[t][e] = x[t] . router[e] (+ bias[e])   MFMA, fp32 accumulate
//   k_topk_dispatch  per tile of 256 tokens: fp32 sigmoid score, top-K by
//                    wave-wide argmax (equal scores: lower expert index), weights
//                    s / sum(s) over the K selected, then a per-expert bitmask of
//                    the tile's tokens gives each pair its rank among earlier
//                    tokens of the tile and the tile's per-expert histogram.
//                    When the whole batch is one tile the same work-group also
//                    scans the counts, scatters the permutation and writes the
//                    expert kernels' tile lists.
//   k_dispatch_scan  (more than one tile) column scan of the tile histograms,
//                    expert offsets, tile lists.
//   k_dispatch_scatter (more than one tile) slot = offset + tile base + rank.
#include <climits>

#include "gemm_core.hpp"
#include "launch.hpp"

namespace flint {

// ---------------------------------------------------------------------------
// Router logits.  SPLITK: 4 waves compute the same 16x16 tile over quarters of
// H (many small work-groups: the decode case, where reading the 1 MiB router
// matrix quickly matters more than reuse).  Otherwise 4 waves in a 2x2 grid,
// each (MB*16) tokens x (NB*16) experts over all of H.
template <typename DT, int MB, int NB, bool SPLITK>
__global__ __launch_bounds__(256) void k_router_logits(const typename DT::storage *__restrict__ x, int T, int H,
                                                       const typename DT::storage *__restrict__ router,
                                                       const float *__restrict__ bias, int E,
                                                       float *__restrict__ z)
{
    using S = typename DT::storage;
    constexpr int WM = SPLITK ? 1 : 2, WN = SPLITK ? 1 : 2;
    constexpr int TILE_T = WM * MB * 16, TILE_E = WN * NB * 16;
    __shared__ float red[SPLITK ? 4 * MB * NB * 256 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = SPLITK ? 0 : wave / WN, wn = SPLITK ? 0 : wave % WN;
    const int t0 = blockIdx.y * TILE_T + wm * MB * 16;
    const int e0 = blockIdx.x * TILE_E + wn * NB * 16;
    const int kg = (lane >> 4) * 8;

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
    const int nslices = H / 32;
    int s0 = 0, s1 = nslices;
    if (SPLITK) {
        const int per = (nslices + 3) / 4;
        s0 = min(wave * per, nslices);
        s1 = min(s0 + per, nslices);
    }
    wave_gemm<DT, MB, NB, 4>(a_rows, b_rows, s0, s1, acc);
    if (SPLITK) {
        splitk_reduce4(acc, red);
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

hipError_t launch_router_logits(bool bf16, const void *x, int T, int H, const void *router,
                                const float *bias, int E, float *logits, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    if (T < 1024) {
        dim3 grid((E + 15) / 16, (T + 15) / 16);
        if (bf16)
            k_router_logits<BF16, 1, 1, true><<<grid, 256, 0, stream>>>(
                (const uint16_t *)x, T, H, (const uint16_t *)router, bias, E, logits);
        else
            k_router_logits<F32, 1, 1, true><<<grid, 256, 0, stream>>>(
                (const float *)x, T, H, (const float *)router, bias, E, logits);
    } else {
        dim3 grid((E + 127) / 128, (T + 63) / 64);
        if (bf16)
            k_router_logits<BF16, 2, 4, false><<<grid, 256, 0, stream>>>(
                (const uint16_t *)x, T, H, (const uint16_t *)router, bias, E, logits);
        else
            k_router_logits<F32, 2, 4, false><<<grid, 256, 0, stream>>>(
                (const float *)x, T, H, (const float *)router, bias, E, logits);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one int per thread over the first 256 threads
// (threads beyond 256 contribute 0).  Every thread of the block must call it.
__device__ int block_exclusive_scan256(int v, int *lds8, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x >= 256) v = 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63 && wave < 4) lds8[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < 4 && w < wave; ++w) base += lds8[w];
    *total = lds8[0] + lds8[1] + lds8[2] + lds8[3];
    __syncthreads();
    return base + incl - v;
}

// Counts -> offsets and the expert kernels' tile lists.  Thread e < E holds
// counts[e] in `c`.  lists: entry i = (expert, first slot of the tile).
__device__ void finish_offsets_and_lists(int c, int E, int32_t *offsets, int32_t *counts,
                                         int32_t *list1, int bm1, int32_t *list2, int bm2,
                                         int32_t *meta, int *lds8)
{
    const int e = threadIdx.x;
    const bool own = e < E;
    if (!own) c = 0;
    int total;
    const int off = block_exclusive_scan256(c, lds8, &total);
    const int n1 = (c + bm1 - 1) / bm1, n2 = (c + bm2 - 1) / bm2;
    int tot1, tot2;
    const int st1 = block_exclusive_scan256(n1, lds8, &tot1);
    const int st2 = block_exclusive_scan256(n2, lds8, &tot2);
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
}

__device__ __forceinline__ float score_from_logit(float z)
{
    // float32 score, rounded once from a double-precision sigmoid.
    return (float)(1.0 / (1.0 + exp(-(double)z)));
}

// One work-group of 1024 threads per tile of 256 tokens.
__global__ __launch_bounds__(1024) void k_topk_dispatch(DispatchArgs a, int fused_single_tile)
{
    __shared__ int16_t sel[kTopkTile * kMaxTopK];
    __shared__ uint32_t masks[kMaxExperts * (kTopkTile / 32)];
    __shared__ int lds8[8];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int E = a.E, K = a.K;
    const int tile = blockIdx.x;
    const int t_base = tile * kTopkTile;
    const int tile_len = min(kTopkTile, a.T - t_base);

    if (a.compute_topk) {
        for (int tl = wave; tl < tile_len; tl += nwaves) {
            const int t = t_base + tl;
            const float *zt = a.logits + (size_t)t * E;
            float s[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                s[j] = e < E ? score_from_logit(zt[e]) : -1.0f;
            }
            unsigned taken = 0;
            int sel_e[kMaxTopK];
            float sel_s[kMaxTopK];
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                sel_e[k] = INT_MAX;
                sel_s[k] = 0.f;
                if (k < K) {
                    float bs = -2.0f;
                    int be = INT_MAX;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // the lane's experts ascend with j, so strict '>' keeps the lower index
                        if (!((taken >> j) & 1u) && s[j] > bs) {
                            bs = s[j];
                            be = lane + 64 * j;
                        }
                    }
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) {
                        const float os = __shfl_xor(bs, off, 64);
                        const int oe = __shfl_xor(be, off, 64);
                        if (os > bs || (os == bs && oe < be)) {
                            bs = os;
                            be = oe;
                        }
                    }
                    sel_e[k] = be;
                    sel_s[k] = bs;
                    if ((be & 63) == lane) taken |= 1u << (be >> 6);
                }
            }
            // ascending expert order (K <= 8; every lane holds the same lists)
#pragma unroll
            for (int i = 1; i < kMaxTopK; ++i)
#pragma unroll
                for (int j = i; j > 0; --j)
                    if (sel_e[j] < sel_e[j - 1]) {
                        const int te = sel_e[j];
                        sel_e[j] = sel_e[j - 1];
                        sel_e[j - 1] = te;
                        const float ts = sel_s[j];
                        sel_s[j] = sel_s[j - 1];
                        sel_s[j - 1] = ts;
                    }
            double sum = 0.0;
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k)
                if (k < K) sum += (double)sel_s[k];
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k)
                if (k < K && lane == k) {
                    a.topk_idx[(size_t)t * K + k] = sel_e[k];
                    a.topk_w[(size_t)t * K + k] = (float)((double)sel_s[k] / sum);
                    sel[tl * K + k] = (int16_t)sel_e[k];
                }
        }
    } else if (a.dispatch) {
        for (int i = threadIdx.x; i < tile_len * K; i += blockDim.x)
            sel[i] = (int16_t)a.topk_idx[(size_t)t_base * K + i];
    }
    if (!a.dispatch) return;

    constexpr int W = kTopkTile / 32;
    for (int i = threadIdx.x; i < E * W; i += blockDim.x) masks[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < tile_len * K; i += blockDim.x) {
        const int tl = i / K, e = sel[i];
        atomicOr(&masks[e * W + (tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    // rank of each (token, expert) pair among the tile's earlier tokens of that expert
    int my_rank[2];
    int my_e[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i = threadIdx.x + r * 1024;
        my_e[r] = -1;
        if (i < tile_len * K) {
            const int tl = i / K, e = sel[i];
            int rk = __popc(masks[e * W + (tl >> 5)] & ((1u << (tl & 31)) - 1u));
            for (int w = 0; w < (tl >> 5); ++w) rk += __popc(masks[e * W + w]);
            my_rank[r] = rk;
            my_e[r] = e;
        }
    }
    int hcount = 0;
    if (threadIdx.x < E)
        for (int w = 0; w < W; ++w) hcount += __popc(masks[threadIdx.x * W + w]);

    if (!fused_single_tile) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = threadIdx.x + r * 1024;
            if (my_e[r] >= 0) a.rank[(size_t)t_base * K + i] = my_rank[r];
        }
        if (threadIdx.x < E) a.hist[(size_t)tile * E + threadIdx.x] = hcount;
        return;
    }

    // Single tile: finish the dispatch here.
    __shared__ int32_t offs[kMaxExperts];
    finish_offsets_and_lists(hcount, E, a.offsets, a.counts, a.list1, a.bm1, a.list2, a.bm2,
                             a.meta, lds8);
    if (threadIdx.x < E) offs[threadIdx.x] = a.offsets[threadIdx.x];
    // offsets were written by this block; re-read through LDS after a barrier
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i = threadIdx.x + r * 1024;
        if (my_e[r] >= 0) {
            const int slot = offs[my_e[r]] + my_rank[r];
            a.sorted_token[slot] = t_base + i / K;
            a.slot_of[(size_t)t_base * K + i] = slot;
        }
    }
}

// More than one tile: per-expert column scan of the tile histograms.
__global__ __launch_bounds__(256) void k_dispatch_scan(DispatchArgs a, int ntiles)
{
    __shared__ int lds8[8];
    const int e = threadIdx.x;
    int run = 0;
    if (e < a.E) {
        for (int tile = 0; tile < ntiles; tile += 8) {
            int h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = tile + j < ntiles ? a.hist[(size_t)(tile + j) * a.E + e] : 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (tile + j < ntiles) a.tile_base[(size_t)(tile + j) * a.E + e] = run;
                run += h[j];
            }
        }
    }
    finish_offsets_and_lists(run, a.E, a.offsets, a.counts, a.list1, a.bm1, a.list2, a.bm2,
                             a.meta, lds8);
}

__global__ __launch_bounds__(256) void k_dispatch_scatter(DispatchArgs a)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.T * a.K) return;
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

hipError_t launch_topk_dispatch(const DispatchArgs &a, hipStream_t stream)
{
    if (a.T <= 0) {
        return hipSuccess;
    }
    const int ntiles = (a.T + kTopkTile - 1) / kTopkTile;
    const int fused = (ntiles == 1) ? 1 : 0;
    k_topk_dispatch<<<ntiles, 1024, 0, stream>>>(a, fused);
    if (a.dispatch && !fused) {
        k_dispatch_scan<<<1, 256, 0, stream>>>(a, ntiles);
        k_dispatch_scatter<<<(a.T * a.K + 255) / 256, 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace flint
