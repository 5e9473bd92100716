// Persistent fused decode layer: top-k, dispatch, gate/up + SwiGLU and down
// for small batches in one launch, the expert work ordered by data flow
// (the release news page, "Built with the Eureka Machine", describes a
// megakernel that fuses the decode forward pass on Apple chips; this is the
// same idea on gfx950).
//
// Layer (serving-kit review, "The architecture, from the config"; release news
// page, "What runs on each token"): K of E experts per token by normalised
// sigmoid scores, each a gated three-matrix SwiGLU of width I, plus an
// always-on shared expert of width Is.
//
// Work units: the shared expert cut into Is / I slices of width I (slice s
// writes the partial output y_shared[s], which the combine adds), and every
// routed expert some token selected.  Unit u belongs to queue u % 8 (shared
// slices first, then the selected experts in ascending order), so the queues
// hold equal numbers of units, i.e. equal weight bytes.  A work-group of class
// q = blockIdx % 8 takes items from queue q, in this order:
//   top-k items      4 tokens each (every queue selects all tokens, so that
//                    no queue waits on another);
//   gate/up items    16 rows x 16 channels of gate and of up of one unit,
//                    the four waves splitting the reduction (H);
//   down items       32 rows x 32 output columns of one unit, the waves
//                    splitting the reduction (I).
// Items are claimed from the queue's counter (relaxed atomics): two
// consecutive ones when a work-group starts, then one at a time, each claimed
// an item ahead of its use.  A work-group whose queue has run out takes
// items from the queue with the most items left (it knows every queue's
// item count from its dispatch and reads the eight claim counters at once),
// so every queue ends at about the same time.
// Dependencies: a unit's gate/up items need the dispatch (all of a queue's
// top-k items done; every work-group then builds the dispatch in its own LDS),
// except the shared slices', which need nothing; a unit's down items need all
// of that unit's gate/up items.  Every dependency of an item lies earlier in
// the same queue, and items are claimed in queue order, so an item only ever
// waits for items that running work-groups have claimed: the kernel cannot
// deadlock even when not all of its work-groups are resident (another kernel
// on the GPU, a smaller grid).
//
// Data that crosses work-groups (the per-queue top-k, h) is written with
// agent-coherent (sc1) stores and read with agent-coherent loads, and a
// completion counter is raised only after the writer's stores have been
// acknowledged, so no cache writeback or invalidate is needed.  Waits poll
// the counter with a bounded number of sleeps; a wait that gives up sets a
// flag in the workspace, and the combine then writes NaN to every output, so
// a failure shows in the result instead of hanging the GPU.
//
// The router runs before (its kernel also zeroes the counters), the combine
// after (it adds the K weighted routed rows and the shared slices in order).
#include "gemm_core.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace flint {

namespace {

constexpr int kQ = kFusedQueues;
constexpr int kW = 4;  // waves per work-group
constexpr int kMaxUnits = kMaxExperts + kFusedMaxShared;
constexpr int kUnitsPerQ = (kMaxUnits + kQ - 1) / kQ;
constexpr int kGuRows = 16, kGuCh = 16;    // gate/up item: rows x channels (of gate and of up)
constexpr int kDnRows = 32, kDnCols = 32;  // down item: rows x output columns
constexpr int kGuTilesPerQ = kUnitsPerQ * (kFusedMaxT / kGuRows);
constexpr int kDnTilesPerQ = kUnitsPerQ * (kFusedMaxT / kDnRows);
constexpr int kSleep = 8;            // s_sleep argument between polls (x 64 cycles: ~0.2 us)
constexpr int kSpinLimit = 1 << 18;  // polls before a wait gives up: ~60 ms
constexpr int kSc1 = 16;             // cache-policy bits of an agent-coherent buffer access

// Counter words (int32) in FusedArgs::sync, each on its own 128-byte line.
__device__ __forceinline__ int32_t *claim_ctr(int32_t *s, int q) { return s + q * 32; }
__device__ __forceinline__ int32_t *topk_ctr(int32_t *s, int q) { return s + (kQ + q) * 32; }
__device__ __forceinline__ int32_t *unit_ctr(int32_t *s, int u) { return s + (2 * kQ + u) * 32; }
__device__ __forceinline__ int32_t *fail_flag(int32_t *s) { return s + (2 * kQ + kMaxUnits) * 32; }
static_assert(kFusedSyncWords == (2 * kQ + kMaxUnits + 1) * 32, "counter words");

__device__ __forceinline__ int ld_agent(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int32_t *p, int v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The calling wave waits until *p >= target (lane 0 polls, the wave follows
// its result).  Gives up after kSpinLimit sleeps and raises the fail flag;
// once the flag is up (the result is void anyway) every wait stops early.
__device__ __forceinline__ void wave_wait_ge(const int32_t *p, int target, int32_t *fail)
{
    const int lane = threadIdx.x & 63;
    for (int spins = 0;; ++spins) {
        int v = 0, failed = 0;
        if (lane == 0) {
            v = ld_agent(p);
            if ((spins & 255) == 255) failed = ld_agent(fail);
        }
        v = __builtin_amdgcn_readfirstlane(v);
        if (v >= target || __builtin_amdgcn_readfirstlane(failed)) return;
        if (spins >= kSpinLimit) {
            if (lane == 0) atomicOr(fail, 1);
            return;
        }
        __builtin_amdgcn_s_sleep(kSleep);
    }
}


struct FusedLds {
    // split-k sums of one item: read and written 16 bytes a lane, so 16-byte
    // aligned (a misaligned array cost the kernel a fifth of its time)
    __attribute__((aligned(16))) float red[kW * 2 * 2 * 256];
    uint64_t mask[kMaxExperts];        // tokens of each expert (bit t)
    int32_t offsets[kMaxExperts + 1];  // first slot of each expert
    int16_t sorted_token[kFusedMaxT * kMaxTopK];
    int16_t unit_e[kMaxUnits];         // unit -> expert, or -1 - s for shared slice s
    int32_t gu_list[kGuTilesPerQ];     // this queue's gate/up row tiles: unit * 8 + tile
    int32_t dn_list[kDnTilesPerQ];     // this queue's down row tiles
    int n_gu, n_dn, n_units, ready, claim, list_q, steal_q;
    int n_items[kQ];  // items of each queue
    int scan[2][kW];
    float ls[kW][kMaxTopK];
    int le[kW][kMaxTopK];
};

enum Kind { TOPK = 0, GU = 1, DN = 2, END = 3 };

// One item as a wave sees it.
template <int MB, int NB>
struct FItem {
    const uint16_t *a[MB];  // GU: x rows (already offset by the lane's k group)
    uint32_t aoff[MB];      // DN: byte offsets of h rows in the h buffer (with the k group)
    const uint16_t *b[NB];  // weight rows (with the k group)
    int s0, nbatch;         // first slice of this wave, batches of U slices
    int row0, row_end;      // rows (slots, or tokens for a shared slice)
    int n0;                 // first channel (GU) / output column (DN)
    int unit, shared;       // unit; shared slice (1) or routed expert (0)
    int slice;              // shared slice index
    int need;               // DN: completed gate/up items of the unit it needs
};

}  // namespace

struct FusedArgs {
    ExpertArgs e;
    const float *logits;  // [logit_splits][T][E]
    int logit_splits;
    int32_t *topk_idx;    // [T][K] routing out (queue 0 writes it)
    float *topk_w;        // [T][K]
    int32_t *topk_q;      // [kQ][T][K] each queue's own copy of the selection
    int32_t *sync;        // kFusedSyncWords counters, zero at launch
    int32_t *counts, *offsets, *sorted_token, *slot_of;  // dispatch out (work-group 0 writes it)
    int n_sh;             // shared slices (Is / I)
};

template <int UG, int UD>
__global__ __launch_bounds__(256, 2) void k_fused_decode(FusedArgs f)
{
    __shared__ FusedLds L;
    const ExpertArgs &a = f.e;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int q = blockIdx.x % kQ;  // the queue this work-group takes items from (uniform)
    const int q0 = q;
    const int T = a.T, H = a.H, E = a.E, K = a.K, I = a.I, Is = a.Is;
    const int n_topk = (T + kW - 1) / kW;
    const int ntn_gu = I / kGuCh, ntn_dn = H / kDnCols;
    const int kg = (lane >> 4) * 8;
    // gate/up items of queue qq's shared slice (unit qq, when qq < n_sh): known
    // before the dispatch
    auto pre_gu_of = [&](int qq) { return qq < f.n_sh ? (T + kGuRows - 1) / kGuRows * ntn_gu : 0; };
    int32_t *const fail = fail_flag(f.sync);
    const __amdgpu_buffer_rsrc_t h_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.h_sorted, 0, (int)((size_t)T * K * I * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t hs_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.h_shared, 0, (int)((size_t)T * (Is > 0 ? Is : 1) * 2), 0x00020000);
    if (tid == 0) {
        L.ready = 0;
        L.list_q = -1;
        L.claim = add_agent(claim_ctr(f.sync, q), 2);  // this work-group's first two items
    }
    __syncthreads();

    // ---- the dispatch, built in this work-group's LDS once it is needed ----
    auto unit_rows = [&](int u) {
        const int e = L.unit_e[u];
        return e < 0 ? T : __popcll(L.mask[e]);
    };
    // the dispatch (the same from every queue's copy of the selection: this
    // work-group's own queue's)
    auto ensure_dispatch = [&]() {
        if (L.ready) return;  // (uniform: read after a barrier)
        if (wave == 0) wave_wait_ge(topk_ctr(f.sync, q0), n_topk, fail);
        __syncthreads();
        const int32_t *sel = f.topk_q + (size_t)q0 * T * K;
        for (int e = tid; e < E; e += 256) L.mask[e] = 0;
        __syncthreads();
        for (int i = tid; i < T * K; i += 256) {
            int e = ld_agent(sel + i);
            if ((unsigned)e >= (unsigned)E) e = 0;  // (only after a wait gave up: the result is void then)
            atomicOr((unsigned long long *)&L.mask[e], 1ull << (i / K));
        }
        __syncthreads();
        // expert counts -> first slots; selected experts -> units (block scan)
        const int cnt = tid < E ? __popcll(L.mask[tid]) : 0, act = cnt > 0;
        int inc0 = cnt, inc1 = act;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y0 = __shfl_up(inc0, off, 64), y1 = __shfl_up(inc1, off, 64);
            if (lane >= off) {
                inc0 += y0;
                inc1 += y1;
            }
        }
        if (lane == 63) {
            L.scan[0][wave] = inc0;
            L.scan[1][wave] = inc1;
        }
        __syncthreads();
        int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
        for (int w = 0; w < kW; ++w) {
            if (w < wave) {
                b0 += L.scan[0][w];
                b1 += L.scan[1][w];
            }
            t0 += L.scan[0][w];
            t1 += L.scan[1][w];
        }
        const int off = b0 + inc0 - cnt, aidx = b1 + inc1 - act;
        if (tid < E) L.offsets[tid] = off;
        if (tid == 0) {
            L.offsets[E] = t0;
            L.n_units = f.n_sh + t1;
        }
        if (tid < f.n_sh) L.unit_e[tid] = (int16_t)(-1 - tid);
        if (act) L.unit_e[f.n_sh + aidx] = (int16_t)tid;
        if (blockIdx.x == 0 && tid < E) {
            f.counts[tid] = cnt;
            f.offsets[tid] = off;
            if (tid == 0) f.offsets[E] = t0;
        }
        __syncthreads();
        // expert-major, token-ascending slots
        for (int i = tid; i < T * K; i += 256) {
            int e = ld_agent(sel + i);
            const int t = i / K;
            if ((unsigned)e >= (unsigned)E) e = 0;
            const int slot = L.offsets[e] + __popcll(L.mask[e] & ((1ull << t) - 1ull));
            L.sorted_token[slot] = (int16_t)t;
            if (blockIdx.x == 0) {
                f.sorted_token[slot] = t;
                f.slot_of[i] = slot;
            }
        }
        __syncthreads();
        if (tid < kQ) {  // items of each queue
            int n = n_topk;
            for (int u = tid; u < L.n_units; u += kQ) {
                const int R = unit_rows(u);
                n += (R + kGuRows - 1) / kGuRows * ntn_gu + (R + kDnRows - 1) / kDnRows * ntn_dn;
            }
            L.n_items[tid] = n;
        }
        if (tid == 0) L.ready = 1;
        __syncthreads();
    };
    // the current queue's row tiles, unit by unit, in LDS
    auto ensure_lists = [&]() {
        ensure_dispatch();
        if (L.list_q == q) return;  // (uniform: read after a barrier)
        __syncthreads();  // every wave is done with the old lists
        if (tid == 0) {
            int ng = 0, nd = 0;
            for (int u = q; u < L.n_units; u += kQ) {
                const int R = unit_rows(u);
                for (int tl = 0; tl * kGuRows < R; ++tl) L.gu_list[ng++] = u * 8 + tl;
                for (int tl = 0; tl * kDnRows < R; ++tl) L.dn_list[nd++] = u * 8 + tl;
            }
            L.n_gu = ng;
            L.n_dn = nd;
            L.list_q = q;
        }
        __syncthreads();
    };
    auto kind_of = [&](int idx) {
        if (idx < n_topk) return (int)TOPK;
        if (idx < n_topk + pre_gu_of(q)) return (int)GU;
        ensure_lists();
        const int end_gu = n_topk + L.n_gu * ntn_gu;
        if (idx < end_gu) return (int)GU;
        if (idx < end_gu + L.n_dn * ntn_dn) return (int)DN;
        return (int)END;
    };

    // ---- items ----
    auto get_gu = [&](int idx) {
        FItem<1, 2> it;
        const int r = idx - n_topk, entry = r / ntn_gu, nt = r % ntn_gu;
        int u, tile;
        if (r < pre_gu_of(q)) {  // this queue's shared slice, before the dispatch is known
            u = q;
            tile = entry;
        } else {
            u = L.gu_list[entry] >> 3;
            tile = L.gu_list[entry] & 7;
        }
        it.unit = u;
        it.shared = u < f.n_sh;
        it.slice = u;
        const int e = it.shared ? 0 : L.unit_e[u];
        const int base = it.shared ? 0 : L.offsets[e];
        const int R = it.shared ? T : __popcll(L.mask[e]);
        it.row0 = base + tile * kGuRows;
        it.row_end = base + R;
        it.n0 = nt * kGuCh;  // channel within the unit
        const int per = H / 32 / kW;
        it.s0 = wave * per;
        it.nbatch = per / UG;
        const uint16_t *wg, *wu;
        if (it.shared) {
            wg = (const uint16_t *)a.shared_gate + (size_t)u * I * H;  // rows s*I.. of [Is][H]
            wu = (const uint16_t *)a.shared_up + (size_t)u * I * H;
        } else {
            wg = (const uint16_t *)a.gate + (size_t)e * I * H;
            wu = (const uint16_t *)a.up + (size_t)e * I * H;
        }
        const int c = it.n0 + (lane & 15);
        it.b[0] = wg + (size_t)c * H + kg;
        it.b[1] = wu + (size_t)c * H + kg;
        int rr = it.row0 + (lane & 15);
        if (rr >= it.row_end) rr = it.row0;  // padded rows repeat the first row
        const int tok = it.shared ? rr : L.sorted_token[rr];
        it.a[0] = (const uint16_t *)a.x + (size_t)tok * H + kg;
        it.aoff[0] = 0;
        it.need = 0;
        return it;
    };
    auto get_dn = [&](int idx) {
        FItem<2, 2> it;
        const int r = idx - n_topk - L.n_gu * ntn_gu, entry = r / ntn_dn, nt = r % ntn_dn;
        const int u = L.dn_list[entry] >> 3, tile = L.dn_list[entry] & 7;
        it.unit = u;
        it.shared = u < f.n_sh;
        it.slice = u;
        const int e = it.shared ? 0 : L.unit_e[u];
        const int base = it.shared ? 0 : L.offsets[e];
        const int R = it.shared ? T : __popcll(L.mask[e]);
        it.row0 = base + tile * kDnRows;
        it.row_end = base + R;
        it.n0 = nt * kDnCols;
        it.need = (R + kGuRows - 1) / kGuRows * ntn_gu;
        const int per = I / 32 / kW;
        it.s0 = wave * per;
        it.nbatch = per / UD;
        // weights: down [E][H][I], or the shared down [H][Is] from column s*I
        const uint16_t *wd = it.shared ? (const uint16_t *)a.shared_down + (size_t)u * I
                                       : (const uint16_t *)a.down + (size_t)e * H * I;
        const int ldw = it.shared ? Is : I;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int c = it.n0 + n * 16 + (lane & 15);
            it.b[n] = wd + (size_t)c * ldw + kg;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            int rr = it.row0 + m * 16 + (lane & 15);
            if (rr >= it.row_end) rr = it.row0;
            it.aoff[m] = it.shared ? (uint32_t)(((size_t)rr * Is + (size_t)u * I + kg) * 2)
                                   : (uint32_t)(((size_t)rr * I + kg) * 2);
            it.a[m] = nullptr;
        }
        return it;
    };

    // claims: the item after `nxt` is claimed while `cur` runs (thread 0), and
    // handed to the work-group at the item's end, after a barrier
    int cur = L.claim, nxt = L.claim + 1, my_claim = 0;
    auto claim_issue = [&]() {
        if (tid == 0) my_claim = add_agent(claim_ctr(f.sync, q), 1);
    };
    auto claim_take = [&]() {
        if (tid == 0) L.claim = my_claim;
        __syncthreads();
        cur = nxt;
        nxt = L.claim;
    };

    // ---- top-k item: tokens 4*idx + wave ----
    auto topk_item = [&](int idx) {
        const int t = idx * kW + wave;
        if (t < T) {
            int sidx;
            float sw;
            wave_topk_select(f.logits + (size_t)t * E, (size_t)T * E, f.logit_splits, E, K, L.ls[wave], L.le[wave],
                             sidx, sw);
            if (lane < K) {
                __hip_atomic_store(f.topk_q + ((size_t)q * T + t) * K + lane, sidx, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (q == 0) {
                    f.topk_idx[(size_t)t * K + lane] = sidx;
                    f.topk_w[(size_t)t * K + lane] = sw;
                }
            }
        }
        wait_vmcnt<0>();  // this wave's stores are acknowledged
        __syncthreads();
        if (tid == 0) add_agent(topk_ctr(f.sync, q), 1);
    };

    // ---- gate/up items (16 x 16 + 16, SwiGLU fused) ----
    auto run_gu = [&]() {
        constexpr int MB = 1, NB = 2, U = UG;
        Frag<BF16> ab[U][NB], aa[U][MB], bb[U][NB], ba[U][MB];
        auto load_batch = [&](const FItem<MB, NB> &it, int batch, Frag<BF16>(&fb)[U][NB], Frag<BF16>(&fa)[U][MB]) {
            const int s = it.s0 + batch * U;
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
#pragma unroll
                for (int n = 0; n < NB; ++n) fb[uu][n].load(it.b[n] + (s + uu) * 32);
#pragma unroll
                for (int m = 0; m < MB; ++m) fa[uu][m].load(it.a[m] + (s + uu) * 32);
            }
        };
        constexpr int kLoadsPerBatch = U * (NB + MB);
        int pending = -1;  // wave 0: unit whose item's h stores must be acknowledged before it is counted
        FItem<MB, NB> it = get_gu(cur);
        load_batch(it, 0, ab, aa);
        while (true) {
            claim_issue();
            const bool next_gu = kind_of(nxt) == GU;
            const FItem<MB, NB> nx = next_gu ? get_gu(nxt) : it;  // (a dummy reload of valid addresses)
            f32x4 acc[MB][NB];
            zero_acc(acc);
            for (int j = 0; j < it.nbatch; j += 2) {
                load_batch(it, j + 1, bb, ba);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int uu = 0; uu < U; ++uu)
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int n = 0; n < NB; ++n) mma(acc[m][n], aa[uu][m], ab[uu][n]);
                const bool more = j + 2 < it.nbatch;
                __builtin_amdgcn_sched_barrier(0);
                load_batch(more ? it : nx, more ? j + 2 : 0, ab, aa);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int uu = 0; uu < U; ++uu)
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int n = 0; n < NB; ++n) mma(acc[m][n], ba[uu][m], bb[uu][n]);
                __builtin_amdgcn_sched_barrier(0);
                if (j == 0 && pending >= 0) {
                    // everything issued before this item's second batch -- the
                    // previous item's h stores among it -- has completed
                    wait_vmcnt<kLoadsPerBatch>();
                    if (lane == 0) add_agent(unit_ctr(f.sync, pending), 1);
                    pending = -1;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            splitk_reduce<kW, MB, NB>(acc, L.red);
            if (wave == 0) {  // (one 16-channel block of gate and of up: wave 0 stores it)
                uint16_t *hout = it.shared ? (uint16_t *)a.h_shared : (uint16_t *)a.h_sorted;
                const int width = it.shared ? Is : I;
                const int c = (it.shared ? it.slice * I : 0) + it.n0 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = it.row0 + (lane >> 4) * 4 + i;
                    if (r < it.row_end)
                        __hip_atomic_store(hout + (size_t)r * width + c, f32_to_bf16(swiglu(acc[0][0][i], acc[0][1][i])),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                pending = it.unit;
            }
            claim_take();  // (its barrier also keeps `red` from being overwritten early)
            if (!next_gu) break;
            it = nx;
        }
        if (pending >= 0) {
            wait_vmcnt<0>();
            if (lane == 0) add_agent(unit_ctr(f.sync, pending), 1);
        }
    };

    // ---- down items (32 x 32, float32 out) ----
    auto run_dn = [&]() {
        constexpr int MB = 2, NB = 2, U = UD;
        Frag<BF16> ab[U][NB], aa[U][MB], bb[U][NB], ba[U][MB];
        auto load_batch = [&](const FItem<MB, NB> &it, int batch, Frag<BF16>(&fb)[U][NB], Frag<BF16>(&fa)[U][MB]) {
            const int s = it.s0 + batch * U;
            const __amdgpu_buffer_rsrc_t rs = it.shared ? hs_rsrc : h_rsrc;
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
#pragma unroll
                for (int n = 0; n < NB; ++n) fb[uu][n].load(it.b[n] + (s + uu) * 32);
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    fa[uu][m].v = __builtin_bit_cast(
                        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, it.aoff[m] + (s + uu) * 64, 0, kSc1));
            }
        };
        FItem<MB, NB> it = get_dn(cur);
        wave_wait_ge(unit_ctr(f.sync, it.unit), it.need, fail);
        load_batch(it, 0, ab, aa);
        while (true) {
            claim_issue();
            const bool next_dn = kind_of(nxt) == DN;
            const FItem<MB, NB> nx = next_dn ? get_dn(nxt) : it;
            // the next item's dependency is read now and checked before its
            // prefetch, so the read's latency hides behind this item
            int dep = 0;
            if (next_dn && lane == 0) dep = ld_agent(unit_ctr(f.sync, nx.unit));
            f32x4 acc[MB][NB];
            zero_acc(acc);
            for (int j = 0; j < it.nbatch; j += 2) {
                load_batch(it, j + 1, bb, ba);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int uu = 0; uu < U; ++uu)
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int n = 0; n < NB; ++n) mma(acc[m][n], aa[uu][m], ab[uu][n]);
                const bool more = j + 2 < it.nbatch;
                __builtin_amdgcn_sched_barrier(0);
                if (!more && next_dn && __builtin_amdgcn_readfirstlane(dep) < nx.need)
                    wave_wait_ge(unit_ctr(f.sync, nx.unit), nx.need, fail);
                load_batch(more ? it : nx, more ? j + 2 : 0, ab, aa);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int uu = 0; uu < U; ++uu)
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int n = 0; n < NB; ++n) mma(acc[m][n], ba[uu][m], bb[uu][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
            splitk_reduce<kW, MB, NB>(acc, L.red);
            float *yout = it.shared ? a.y_shared + (size_t)it.slice * T * H : a.y_sorted;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                if (n != wave) continue;  // waves 0 and 1 store a 16-column block each
                const int c = it.n0 + n * 16 + (lane & 15);
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = it.row0 + m * 16 + (lane >> 4) * 4 + i;
                        if (r < it.row_end) yout[(size_t)r * H + c] = acc[m][n][i];
                    }
            }
            claim_take();
            if (!next_dn) break;
            it = nx;
        }
    };

    // the queue with the most items left (thread 0 looks, the work-group
    // follows): claims two items there; false when every queue is empty
    auto steal = [&]() {
        if (tid == 0) {
            L.steal_q = -1;
            for (int tries = 0; tries < 4 && L.steal_q < 0; ++tries) {
                int taken[kQ];
#pragma unroll
                for (int i = 0; i < kQ; ++i) taken[i] = ld_agent(claim_ctr(f.sync, i));
                int qn = -1, most = 0;
#pragma unroll
                for (int i = 0; i < kQ; ++i)
                    if (L.n_items[i] - taken[i] > most) {
                        most = L.n_items[i] - taken[i];
                        qn = i;
                    }
                if (qn < 0) break;
                const int c = add_agent(claim_ctr(f.sync, qn), 2);
                if (c < L.n_items[qn]) {
                    L.steal_q = qn;
                    L.claim = c;
                }
            }
        }
        __syncthreads();
        if (L.steal_q < 0) return false;
        q = L.steal_q;
        cur = L.claim;
        nxt = L.claim + 1;
        return true;
    };

    while (true) {
        const int kind = kind_of(cur);
        if (kind == END) {
            if (!steal()) break;
            continue;
        }
        if (kind == TOPK) {
            claim_issue();
            topk_item(cur);
            claim_take();
        } else if (kind == GU) {
            run_gu();
        } else {
            run_dn();
        }
    }
    if (blockIdx.x == 0) ensure_dispatch();  // work-group 0 writes the dispatch out for the combine
}

// ---------------------------------------------------------------------------

static int fused_unroll(int k)
{
    // each wave a quarter of the reduction, an even number of batches of U slices
    for (int U : {2, 1})
        if (k % (32 * kW * U * 2) == 0) return U;
    return 0;
}

bool fused_eligible(int T, int H, int E, int K, int I, int Is, bool bf16)
{
    if (!bf16 || T < 1 || T > kFusedMaxT || K < 1 || E > kMaxExperts) return false;
    if (I % kGuCh || H % kDnCols || fused_unroll(H) == 0 || fused_unroll(I) == 0) return false;
    if (Is % I || Is / I > kFusedMaxShared) return false;
    return true;
}

hipError_t launch_fused_decode(const ExpertArgs &a, const float *logits, int logit_splits, int32_t *topk_idx,
                               float *topk_w, int32_t *topk_q, int32_t *sync, int32_t *counts, int32_t *offsets,
                               int32_t *sorted_token, int32_t *slot_of, hipStream_t stream, Marks m)
{
    FusedArgs f{};
    f.e = a;
    f.logits = logits;
    f.logit_splits = logit_splits;
    f.topk_idx = topk_idx;
    f.topk_w = topk_w;
    f.topk_q = topk_q;
    f.sync = sync;
    f.counts = counts;
    f.offsets = offsets;
    f.sorted_token = sorted_token;
    f.slot_of = slot_of;
    f.n_sh = a.Is / a.I;
    const int grid = 2 * a.cus / kQ * kQ;  // two work-groups per CU, a multiple of the queue count
    const int ug = fused_unroll(a.H), ud = fused_unroll(a.I);
    if (ug == 2 && ud == 2) return launch_k(k_fused_decode<2, 2>, grid, 256, 0, stream, m, f);
    if (ug == 2) return launch_k(k_fused_decode<2, 1>, grid, 256, 0, stream, m, f);
    if (ud == 2) return launch_k(k_fused_decode<1, 2>, grid, 256, 0, stream, m, f);
    return launch_k(k_fused_decode<1, 1>, grid, 256, 0, stream, m, f);
}

}  // namespace flint
