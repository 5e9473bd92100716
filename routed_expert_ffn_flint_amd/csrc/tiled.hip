// LDS-tiled GEMMs: the grouped expert products and the router for large
// batches (prefill), and a dense bf16 layer's products at every batch size.
//
// Layer (serving-kit review, "The architecture, from the config"; release news
// page, "What runs on each token"): a sigmoid router over the experts, then K
// selected experts of width I per token plus an always-on shared expert of
// width Is, each a gated three-matrix SwiGLU.
//
// With hundreds of rows per expert the expert products are real GEMMs, so both
// operands are staged through LDS and reused:
//   - a work-group computes a BM x BN output tile; its waves each own a
//     WM x WN block built from 16x16x32 bf16 MFMAs; k runs in slices of BK =
//     32 or 64 (per configuration);
//   - operands go from global memory straight into LDS
//     (global_load_lds_dwordx4: lane l of a wave's load lands at the
//     instruction's LDS base + 16 l), so no registers hold them in flight and
//     no LDS write instructions are issued;
//   - a stage holds the tile's BM A rows then its BN B rows, 2 BK bytes each.
//     The 16-byte chunk c of row r is stored at chunk position c ^ (r & 7)
//     (BK = 64: a load instruction covers 8 whole rows, each one 128-byte
//     global segment) or c ^ ((r >> 1) & 3) (BK = 32: 16 rows of 64 bytes), so
//     a fragment read -- 16 rows, one chunk -- touches 16 distinct bank groups;
//   - slice s is fetched into stage s % STAGES at the end of iteration
//     s - STAGES (the first STAGES slices before the loop), so STAGES - 1
//     slices are in flight behind the MFMA work.  One barrier per iteration,
//     at the last step of slice kt: after it every wave's share of slice kt+1
//     has landed (each wave waits for its own first), and every wave holds
//     slice kt's last fragments in registers, so stage kt % STAGES is free
//     for slice kt + STAGES.  The stages are separate LDS arrays and the
//     waits explicit; fetches past the last slice re-read it, into stages
//     never read again, so the number of loads in flight at each wait is the
//     same every iteration (refilling the stage just read, instead of the one
//     read an iteration earlier, keeps one more slice in flight: T = 4096
//     gate/up 285 -> 259 us, down 184 -> 177 us on 128 x 256 tiles);
//   - gate/up tiles hold BN/2 gate rows and the BN/2 up rows of the same
//     channels; each wave's columns are WN/2 gate + the matching WN/2 up
//     channels, so silu(g) * u is formed in registers;
//   - routed rows are gathered through the expert-sorted token list;
//   - work items are (expert tile, n-tile) with n fastest; XCD j runs the j-th
//     eighth of the items, in order, so the n-tiles of one expert tile (which
//     gather the same rows) and consecutive expert tiles (same weights) share
//     that XCD's L2.  Shared-weight items (the shared expert, the dense layer)
//     go n-tile outer over groups of 8 row tiles, so that both operands repeat
//     in L2 (dense T = 4096 gate/up: 251 -> 235 us; its L2 misses had been
//     14x the algorithmic bytes).  The down product deals each XCD an eighth
//     of the shared and an eighth of the routed items;
//   - waves whose rows are all padding (an expert's last tile) only fetch
//     their share and keep the barriers;
//   - a dense layer's down product splits its reduction over the width into
//     partial arrays (the combine adds them) to fill the CUs.
#include "gemm_core.hpp"
#include "launch.hpp"
#include "tile_sched.hpp"

namespace flint {

namespace {

constexpr int kLdsBytes = 160 * 1024;

// Tile configuration: work-group tile BM x BN, wave tile WM x WN, k slice BK
// (32 or 64) per LDS stage, STAGES stages.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_;
    static constexpr int WAVES_N = BN / WN, WAVES = (BM / WM) * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int MB = WM / 16, NB = WN / 16;
    static constexpr int CPR = BK / 8;               // 16-byte chunks per LDS row
    static constexpr int ROWS_PER_LOAD = 64 / CPR;   // rows one load instruction covers
    static constexpr int NQ = BK / 32;               // 32-wide MFMA steps per slice
    static constexpr int STAGE_ELEMS = (BM + BN) * BK;
    static constexpr int LOADS_A = BM / ROWS_PER_LOAD / WAVES, LOADS_B = BN / ROWS_PER_LOAD / WAVES;
    static constexpr int LDS = STAGES * STAGE_ELEMS * 2;
    static constexpr int WGS_PER_CU = kLdsBytes / LDS >= 2 ? 2 : 1;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 16 == 0 && WN % 32 == 0, "tile shape");
    static_assert(BK == 32 || BK == 64, "slice");
    static_assert(LOADS_A * ROWS_PER_LOAD * WAVES == BM && LOADS_B * ROWS_PER_LOAD * WAVES == BN, "rows per wave");
    static_assert(STAGES >= 3 && STAGES <= 8 && LDS <= kLdsBytes, "stages");
    // slices per unrolled round: stage index and fragment-buffer parity both static
    static constexpr int ROUND = (NQ == 1 && STAGES % 2) ? 2 * STAGES : STAGES;
    // stored chunk position of logical chunk c in row r
    __device__ static __forceinline__ int swz(int r, int c) { return CPR == 8 ? c ^ (r & 7) : c ^ ((r >> 1) & 3); }
};

// Configurations (chosen per launch by the host).
// Cfg<BM, BN, WM, WN, BK, STAGES>; the 128 x 256 tiles take 64-wide slices
// in 3 stages (T = 4096: 570 -> 560 us against 32-wide slices in 4).
using CfgSmall = Cfg<128, 128, 64, 64, 32, 5>;  // 4 waves
using CfgWide = Cfg<256, 128, 128, 64, 32, 6>;  // 4 waves
using CfgBig = Cfg<256, 256, 128, 128, 32, 4>;  // 4 waves
using CfgBig8 = Cfg<256, 256, 128, 64, 32, 4>;  // 8 waves
using CfgWideN = Cfg<128, 256, 64, 64, 64, 3>;  // 8 waves
// A routed layer of a few dozen rows per expert: 64-row tiles in 4 stages (the
// whole LDS), so less of each tile is padding and more of the weights are in
// flight per CU.  Layer times on the Flint shape (H = 2048, 256 experts, top 6,
// widths 512 / 1024) against the 128 x 256 tiles: T = 640 374 -> 363 us,
// 1024 387 -> 375 (gate/up and down on 64-row tiles), 1536 407 -> 396 (gate/up
// only); slower from 48 rows per expert (T = 2048: gate/up 230 -> 244 us, down
// on them from 36 rows: 127 -> 132).  CfgMidN: widths not whole 128-channel tiles.
using CfgMid = Cfg<64, 256, 32, 64, 64, 4>;   // 8 waves
using CfgMidN = Cfg<64, 128, 32, 64, 64, 4>;  // 4 waves
// The router from T = 1024 on: 64 tokens x all 256 experts, so each token row
// is read from HBM once and the 1 MiB router matrix (read by every row tile)
// from L2 (T = 1024 16.7 -> 12.7 us, 4096 19.3 -> 15.1, 16384 39.9 -> 35.6
// against 128 x 128 tiles; 32 x 256 tiles on 4 waves 12.6, 25.4, 60.9).
using CfgRouter = Cfg<64, 256, 32, 64, 64, 3>;  // 8 waves
// A dense layer at decode sizes (T < kDenseTiledFromT): 32-row tiles and
// rings of 64-wide slices, the weights streaming through LDS with several
// slices in flight per work-group; gate/up 32 gate + 32 up channels on two
// waves (6 stages, two work-groups per CU, up to 64 rows; beyond, 4 stages and
// three per CU for the extra row tiles: T = 128 gate/up 31.8 -> 24.1 us, T = 64
// 18.3 -> 19.0), down 64 columns on one wave over a split of the width.
using CfgDecGu = Cfg<32, 64, 32, 32, 64, 6>;    // 2 waves
using CfgDecGu4 = Cfg<32, 64, 32, 32, 64, 4>;   // 2 waves
using CfgDecDn = Cfg<32, 64, 32, 64, 64, 6>;    // 1 wave
constexpr int kDecGuRows6 = 64;  // largest batch on CfgDecGu
// A MoE layer below kLargeTilesFromT rows (a few to a few dozen rows per
// expert): 16-row tiles, so an expert's rows waste little of a tile; gate/up
// 32 gate + 32 up channels on two waves (6 stages, two work-groups per CU),
// down 128 columns on two waves (4 stages).  Measured at T = 256 (Flint shape)
// against 32-row tiles: gate/up 191 vs 198 us, down 111 vs 127; down on
// 64-column items 110-121 us, 6 stages 121.
using CfgMoeGu = Cfg<16, 64, 16, 32, 64, 6>;   // 2 waves
using CfgMoeDn = Cfg<16, 128, 16, 64, 64, 4>;  // 2 waves

enum Mode { GATE_UP = 0, DOWN = 1, ROUTER = 2 };

// The largest of v over each row of 16 lanes (lanes 16k .. 16k+15), in every
// lane of the row: DPP swaps within quads, then the mirrors of 8 and of 16
// lanes (VALU operations, no LDS traffic).
__device__ __forceinline__ float row16_max(float v)
{
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
    return v;
}

}  // namespace

struct TiledArgs {
    ExpertArgs e;
    int n_shared;        // shared-expert items (they come first)
    int ksplit;          // ROUTER: partial sums over this many slices of H
    const void *router;  // ROUTER: [E][H]
    const float *bias;   // ROUTER: [E] or null
    float *logits;       // ROUTER: [T][E]
};

template <int MODE, typename C>
__global__ __launch_bounds__(C::THREADS, C::WGS_PER_CU) void k_tiled(TiledArgs ta)
{
    using S = uint16_t;
    constexpr int BM = C::BM, BN = C::BN, MB = C::MB, NB = C::NB, STAGES = C::STAGES;
    // one LDS array per stage (separate objects, so the compiler can tell the
    // stage being filled from the stage being read)
    __shared__ __attribute__((aligned(16))) S st0[C::STAGE_ELEMS];
    __shared__ __attribute__((aligned(16))) S st1[C::STAGE_ELEMS];
    __shared__ __attribute__((aligned(16))) S st2[C::STAGE_ELEMS];
    __shared__ __attribute__((aligned(16))) S st3[STAGES > 3 ? C::STAGE_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) S st4[STAGES > 4 ? C::STAGE_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) S st5[STAGES > 5 ? C::STAGE_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) S st6[STAGES > 6 ? C::STAGE_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) S st7[STAGES > 7 ? C::STAGE_ELEMS : 8];
    auto stage = [&](int i) -> S * {
        return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : i == 3 ? st3 : i == 4 ? st4 : i == 5 ? st5 : i == 6 ? st6 : st7;
    };

    const ExpertArgs &a = ta.e;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int H = a.H;

    // ---- the work item: rows [row0, row_end) of A, n-tile nt, reduction kdim
    // from kbase of rows kstride long
    int row0, row_end, nt, kdim, e = 0;
    bool shared = false;
    int kbase = 0, kstride = 0;
    float *lout = nullptr;
    float *yout = nullptr;  // DOWN: the output array of this item
    if (MODE == ROUTER) {
        const int ntn = (a.E + BN - 1) / BN;
        const int item = xcd_item(((a.T + BM - 1) / BM) * ntn * ta.ksplit);
        if (item < 0) return;
        const int ks = item % ta.ksplit, tile = item / ta.ksplit;
        row0 = (tile / ntn) * BM;
        nt = tile % ntn;
        row_end = a.T;
        kdim = H / ta.ksplit;
        kbase = ks * kdim;
        kstride = H;
        lout = ta.logits + (size_t)ks * a.T * a.E;
        if (ks != 0) ta.bias = nullptr;
    } else {
        const int ntn_shared = MODE == GATE_UP ? a.Is / (BN / 2) : (H + BN - 1) / BN;
        const int ntn_routed = MODE == GATE_UP ? a.I / (BN / 2) : (H + BN - 1) / BN;
        const int nlist = MODE == GATE_UP ? (a.K > 0 ? a.meta[0] : 0) : (a.K > 0 ? a.meta[1] : 0);
        // gate/up: all items cost alike, and contiguous eighths keep the shared
        // expert's weights on one XCD; down: shared items reduce over Is, routed
        // ones over I, so each XCD takes its share of both kinds
        const int item = MODE == GATE_UP ? xcd_item(ta.n_shared + nlist * ntn_routed)
                                         : xcd_item2(ta.n_shared, nlist * ntn_routed);
        if (item < 0) return;
        shared = item < ta.n_shared;
        if (shared) {
            // down: split sp of the reduction over Is (split outermost)
            const int nrt = (a.T + BM - 1) / BM;
            const int sp = MODE == DOWN ? item / (nrt * ntn_shared) : 0;
            const int it = MODE == DOWN ? item % (nrt * ntn_shared) : item;
            // groups of kRowGroup row tiles, n-tile outer within a group: the
            // work-groups running together on an XCD cover a few row tiles and a
            // few n-tiles, and both their rows and their weights repeat in L2
            const int g = it / (kRowGroup * ntn_shared), w = it % (kRowGroup * ntn_shared);
            const int rows_here = min(kRowGroup, nrt - g * kRowGroup);
            row0 = (g * kRowGroup + w % rows_here) * BM;
            nt = w / rows_here;
            row_end = a.T;
            kstride = MODE == GATE_UP ? H : a.Is;
            kdim = MODE == GATE_UP ? H : a.Is / (a.shared_splits > 1 ? a.shared_splits : 1);
            kbase = sp * kdim;
            yout = a.y_shared + (size_t)sp * a.T * H;
        } else {
            const int r = item - ta.n_shared;
            const int entry = r / ntn_routed;
            const int32_t *list = MODE == GATE_UP ? a.list1 : a.list2;
            e = list[2 * entry];
            row0 = list[2 * entry + 1];
            nt = r % ntn_routed;
            row_end = a.offsets[e + 1];
            kdim = kstride = MODE == GATE_UP ? H : a.I;
            yout = a.y_sorted;
        }
    }

    // ---- this lane's fetch sources.  Load instruction i of this wave covers
    // ROWS_PER_LOAD rows of A (or of B); the lane takes row + lane / CPR and
    // the logical chunk whose stored position is lane % CPR.
    constexpr int BK = C::BK, CPR = C::CPR, RPL = C::ROWS_PER_LOAD;
    const S *ga[C::LOADS_A];
    const S *gb[C::LOADS_B];
#pragma unroll
    for (int i = 0; i < C::LOADS_A; ++i) {
        const int rr = (wave * C::LOADS_A + i) * RPL + lane / CPR;
        const int chunk = C::swz(rr, lane % CPR) * 8;  // (the swizzle is its own inverse)
        int r = row0 + rr;
        if (r >= row_end) r = row0;  // padded rows repeat the first row
        if (MODE == GATE_UP) {
            const int tok = shared ? r : a.sorted_token[r];
            ga[i] = (const S *)a.x + (size_t)tok * H + chunk;
        } else if (MODE == DOWN) {
            ga[i] = (shared ? (const S *)a.h_shared : (const S *)a.h_sorted) + (size_t)r * kstride + kbase + chunk;
        } else {
            ga[i] = (const S *)a.x + (size_t)r * H + kbase + chunk;
        }
    }
#pragma unroll
    for (int i = 0; i < C::LOADS_B; ++i) {
        const int rr = (wave * C::LOADS_B + i) * RPL + lane / CPR;
        const int chunk = C::swz(rr, lane % CPR) * 8;
        if (MODE == GATE_UP) {
            // B rows [0, BN/2): gate channels nt*BN/2 + rr; then the same up channels
            const int ch = nt * (BN / 2) + (rr % (BN / 2));
            const bool up = rr >= BN / 2;
            const S *w = shared ? (up ? (const S *)a.shared_up : (const S *)a.shared_gate)
                                : (up ? (const S *)a.up : (const S *)a.gate) + (size_t)e * a.I * H;
            gb[i] = w + (size_t)ch * H + chunk;
        } else if (MODE == DOWN) {
            int c = nt * BN + rr;
            if (c >= H) c = 0;
            const S *w = shared ? (const S *)a.shared_down : (const S *)a.down + (size_t)e * H * a.I;
            gb[i] = w + (size_t)c * kstride + kbase + chunk;
        } else {
            int c = nt * BN + rr;
            if (c >= a.E) c = 0;
            gb[i] = (const S *)ta.router + (size_t)c * H + kbase + chunk;
        }
    }
    auto fetch = [&](S *buf, int k0) {
#pragma unroll
        for (int i = 0; i < C::LOADS_A; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(ga[i] + k0),
                                             LDS_PTR(buf + (wave * C::LOADS_A + i) * RPL * BK), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < C::LOADS_B; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(gb[i] + k0),
                                             LDS_PTR(buf + (BM + (wave * C::LOADS_B + i) * RPL) * BK), 16, 0, 0);
    };
    constexpr int kLoadsPerSlice = C::LOADS_A + C::LOADS_B;

    // ---- fragments: MB row blocks (A) x NB column blocks (B) of 16.
    // A rows: wm*WM + m*16 + (lane&15).  B rows (GATE_UP): gate blocks j < NB/2
    // at wn*WN/2 + j*16, up blocks at BN/2 + wn*WN/2 + (j - NB/2)*16;
    // otherwise wn*WN + j*16.  Every fragment row is congruent to lane & 15
    // mod 16, so its swizzle depends on the lane only.
    int aoff[MB], boff[NB];
#pragma unroll
    for (int m = 0; m < MB; ++m) aoff[m] = (wm * C::WM + m * 16 + (lane & 15)) * BK;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int br = MODE == GATE_UP ? (j < NB / 2 ? wn * (C::WN / 2) + j * 16
                                                     : BN / 2 + wn * (C::WN / 2) + (j - NB / 2) * 16)
                                       : wn * C::WN + j * 16;
        boff[j] = (BM + br + (lane & 15)) * BK;
    }
    int qoff[C::NQ];  // element offset of this lane's 8 k values in 32-wide step q
#pragma unroll
    for (int q = 0; q < C::NQ; ++q) qoff[q] = C::swz(lane & 15, q * 4 + (lane >> 4)) * 8;

    struct Frags {
        Frag<BF16> a[MB], b[NB];
    };
    auto read = [&](Frags &f, const S *buf, int q) {
#pragma unroll
        for (int m = 0; m < MB; ++m) f.a[m].load(buf + aoff[m] + qoff[q]);
#pragma unroll
        for (int j = 0; j < NB; ++j) f.b[j].load(buf + boff[j] + qoff[q]);
    };
    f32x4 acc[MB][NB];
    auto mmas = [&](const Frags &f) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < NB; ++j) mma(acc[m][j], f.a[m], f.b[j]);
    };
    // the next step's fragment reads spread over this step's MFMAs
    constexpr int kReads = MB + NB, kMfma = MB * NB, kPer = kMfma / kReads;
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < kReads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);  // kPer MFMAs
        }
        if (kMfma > kPer * kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPer * kReads, 0);
    };

    // ---- main loop.  Step (kt, q) runs the MFMAs of 32-wide step q of slice
    // kt (in stage kt % STAGES) from fragment buffer p while the reads of the
    // next step go to the other buffer.  At the last step of a slice: wait
    // until this lane's part of slice kt+1 has landed, barrier (now all of it
    // has, and every wave has read its last fragments of slice kt), refill
    // slice kt's stage with slice kt+STAGES, and read the first step of slice
    // kt+1.
    zero_acc(acc);
    const int nk = kdim / BK;
    // Down products: each work-group walks k from its own starting slice, so
    // that the work-groups running at once read different columns of their
    // 1 KB rows (measured faster).  Gate/up products keep one order: there the
    // n-tiles of an expert tile read the same gathered rows at the same time,
    // from L2.
    const int rot = MODE == DOWN ? (int)(blockIdx.x * 7u % (unsigned)nk) : 0;
    auto kofs = [&](int s) {
        s = min(s, nk - 1) + rot;
        return (s >= nk ? s - nk : s) * BK;
    };
    Frags fr[2];
    // j: position in the unrolled round (stage j % STAGES).  LIVE: the wave
    // has rows to compute.  A wave whose rows are all padding (the second half
    // of an expert's last tile when at most WM rows are left) only fetches its
    // share of the slices and keeps the barriers, so the MFMA pipes serve the
    // live waves alone.
    auto step = [&](auto live, int j, int q, int kt) {
        constexpr bool LIVE = decltype(live)::value;
        const int p = (j * C::NQ + q) & 1;
        const int st = j % STAGES;
        if (LIVE) wait_lds();  // fr[p] has landed
        __builtin_amdgcn_sched_barrier(0);
        if (q == C::NQ - 1) {
            wait_vmcnt<(STAGES - 2) * kLoadsPerSlice>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            fetch(stage(st), kofs(kt + STAGES));
            __builtin_amdgcn_sched_barrier(0);
            if (LIVE) read(fr[p ^ 1], stage((st + 1) % STAGES), 0);
        } else if (LIVE) {
            read(fr[p ^ 1], stage(st), q + 1);
        }
        if (LIVE) {
            mmas(fr[p]);
            interleave();
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto run = [&](auto live) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) fetch(stage(s), kofs(s));
        wait_vmcnt<(STAGES - 1) * kLoadsPerSlice>();
        __builtin_amdgcn_s_barrier();
        if (decltype(live)::value) read(fr[0], stage(0), 0);
        // whole rounds, with no branch inside (so the compiler keeps its own
        // waits off the LDS reads); then the rest
        constexpr int ROUND = C::ROUND;
        const int nfull = nk / ROUND * ROUND;
        for (int kb = 0; kb < nfull; kb += ROUND) {
#pragma unroll
            for (int j = 0; j < ROUND; ++j)
#pragma unroll
                for (int q = 0; q < C::NQ; ++q) step(live, j, q, kb + j);
        }
#pragma unroll
        for (int j = 0; j + 1 < ROUND; ++j) {
            if (nfull + j >= nk) break;
#pragma unroll
            for (int q = 0; q < C::NQ; ++q) step(live, j, q, nfull + j);
        }
    };
    // waves whose rows all lie past the tile's end skip the MFMAs (they still
    // take part in the loads and barriers)
    if (row0 + wm * C::WM < row_end)
        run(std::integral_constant<bool, true>{});
    else
        run(std::integral_constant<bool, false>{});
    // no load may still be writing this work-group's LDS when it exits
    wait_vmcnt<0>();
    wait_lds();

    // ---- epilogue: lane holds C[(lane>>4)*4 + i][lane&15] of each 16x16 block
    // Routed down rows are stored as fp16 times 2^s, one exponent s per row
    // and 64 columns (four 16-column blocks): s = 0 unless the 64 values'
    // largest magnitude reaches 2^15, then the smallest s that brings it
    // below (so no finite value overflows fp16); the combine multiplies back.
    // The exponents start at 0 (the dispatch clears them); a wave none of
    // whose values reaches 2^15 -- the usual case -- stores none.
    // With 64-column wave tiles the fp16 rows are first gathered in the
    // (by now idle) LDS stages, one wave-tile region per wave, and then
    // written out as 16-byte pieces of whole rows instead of 2-byte scattered
    // stores.
    constexpr int kGroups = (MODE == DOWN) ? NB / 4 : 1;
    static_assert(MODE != DOWN || NB % 4 == 0, "64-column exponent groups");
    // (a routed layer's shared rows too: its tiled path keeps one y_shared array)
    const bool y16 = MODE == DOWN && a.y16 && (!shared || a.shared_splits <= 1);
    // exponent row of output row r: routed slots first, then the shared rows
    const size_t scale_row0 = shared ? (size_t)a.T * a.K : 0;
    constexpr bool kStaged = MODE == DOWN && C::WN == 64;
    constexpr int kWavesPerStage = C::STAGE_ELEMS / (C::WM * C::WN);
    static_assert(!kStaged || C::WAVES <= STAGES * kWavesPerStage, "a wave-tile region of LDS per wave");
    _Float16 *ystage = nullptr;
    bool scaled = false;  // some value of this wave reaches 2^15 (uniform over the wave)
    if (MODE == DOWN && y16) {
        float mx = 0.f;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[m][j][i]));
        scaled = __ballot(!(mx < 32768.0f)) != 0;  // (NaN counts as large: it takes the careful path)
    }
    if (kStaged && y16) {
        __syncthreads();  // every wave is done with the stages
        ystage = reinterpret_cast<_Float16 *>(stage(wave / kWavesPerStage)) + (wave % kWavesPerStage) * C::WM * C::WN;
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = wm * C::WM + m * 16 + (lane >> 4) * 4 + i;
            const int r = row0 + rl;
            int sexp[kGroups];
#pragma unroll
            for (int g = 0; g < kGroups; ++g) sexp[g] = 0;
            if (MODE == DOWN && y16 && scaled) {
#pragma unroll
                for (int g = 0; g < kGroups; ++g) {
                    float mx = 0.f;
#pragma unroll
                    for (int j = 4 * g; j < 4 * g + 4; ++j) mx = fmaxf(mx, fabsf(acc[m][j][i]));
                    mx = row16_max(mx);  // the row's 16 lanes
                    const int e = (int)((__float_as_uint(mx) >> 23) & 255u) - 126;  // mx < 2^e
                    sexp[g] = (mx >= 32768.0f && e <= 128) ? e - 15 : 0;
                }
            }
            if (r >= row_end) continue;
            if (MODE == GATE_UP) {
                S *hout = shared ? (S *)a.h_shared : (S *)a.h_sorted;
                const int width = shared ? a.Is : a.I;
#pragma unroll
                for (int j = 0; j < NB / 2; ++j) {
                    const int ch = nt * (BN / 2) + wn * (C::WN / 2) + j * 16 + (lane & 15);
                    hout[(size_t)r * width + ch] = f32_to_bf16(swiglu(acc[m][j][i], acc[m][j + NB / 2][i]));
                }
            } else if (MODE == DOWN) {
                if (y16) {
                    if (kStaged) {
                        // row rl of the wave tile, 16-byte chunk j*2 + (lane&15)/8 stored at
                        // chunk ^ (row & 7)
                        const int rw = m * 16 + (lane >> 4) * 4 + i;
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            const int col = j * 16 + (lane & 15);
                            const int pc = (col >> 3) ^ (rw & 7);
                            ystage[rw * 64 + pc * 8 + (col & 7)] = (_Float16)ldexpf(acc[m][j][i], -sexp[j / 4]);
                        }
                    } else {
                        _Float16 *y = reinterpret_cast<_Float16 *>(yout);
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            const int c = nt * BN + wn * C::WN + j * 16 + (lane & 15);
                            if (c < H) y[(size_t)r * H + c] = (_Float16)ldexpf(acc[m][j][i], -sexp[j / 4]);
                        }
                    }
#pragma unroll
                    for (int g = 0; g < kGroups; ++g) {
                        const int c = nt * BN + wn * C::WN + g * 64;
                        if (scaled && (lane & 15) == 0 && c < H)
                            a.y_scale[(scale_row0 + r) * (H / kYScaleCols) + c / kYScaleCols] = (int8_t)sexp[g];
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const int c = nt * BN + wn * C::WN + j * 16 + (lane & 15);
                        if (c < H) yout[(size_t)r * H + c] = acc[m][j][i];
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int c = nt * BN + wn * C::WN + j * 16 + (lane & 15);
                    if (c < a.E) lout[(size_t)r * a.E + c] = acc[m][j][i] + (ta.bias ? ta.bias[c] : 0.f);
                }
            }
        }
    }
    if (kStaged && y16) {
        // whole rows out: 8 lanes a row (16 bytes each), 8 rows an instruction
        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
        const int c = nt * BN + wn * C::WN;
        _Float16 *y = reinterpret_cast<_Float16 *>(yout);
#pragma unroll
        for (int p = 0; p < C::WM / 8; ++p) {
            const int rw = p * 8 + lane / 8, c8 = lane % 8;
            const u32x4v v = *reinterpret_cast<const u32x4v *>(ystage + rw * 64 + (c8 ^ (rw & 7)) * 8);
            const int r = row0 + wm * C::WM + rw;
            if (r < row_end && c < H) *reinterpret_cast<u32x4v *>(y + (size_t)r * H + c + c8 * 8) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side

constexpr int kTlBigRows = 256;  // mean rows per expert from which the down product takes 256 x 256 tiles
// Gate/up on 128 x 256 tiles (a routed layer above kTlMidGuRows rows per expert; a dense layer
// unless its 256 x 256 tiles come in fewer waves, see dense_gu_big) (which: 0 CfgSmall, 1 CfgWide,
// 2 CfgBig, 3 CfgBig8, 6 CfgWideN; T = 4096: 290 -> 280 us against CfgSmall;
// T = 16384: 667 -> 625 us against CfgBig8, 879 with CfgBig, 946 with CfgWide).
constexpr int kTlGuWide = 6;
constexpr int kTlDnSmall = 6;  // (T = 2048: 128 x 256 tiles 154 -> 144 us; even at 4096)
constexpr int kTlDnBig = 3;  // (T = 16384: 8 waves measured 3% faster for the layer than 4; 128 x 256: 498 vs 478 us)
// mean rows per expert (T K / E) up to which gate/up (down) takes the 64-row tiles
constexpr int kTlMidGuRows = 40;
constexpr int kTlMidDnRows = 24;
constexpr int kTlMid = 7;

namespace {

// which: 0 CfgSmall, 1 CfgWide, 2 CfgBig, 3 CfgBig8, 6 CfgWideN, 7 CfgMid
int cfg_bm(int which) { return which == kTlMid ? 64 : which >= 1 && which <= 3 ? 256 : 128; }
int cfg_bn(int which) { return which >= 2 ? 256 : 128; }

bool big_batch(int T, int K, int E) { return (long long)T * K >= (long long)kTlBigRows * E; }

// A dense layer (no routed experts) has T rows in every product, so its tiles
// come in whole waves over the 256 CUs of an MI355X (one work-group per CU
// for the 128 x 256 and 256 x 256 tiles).  Gate/up takes the 256 x 256 tiles
// (twice the work per item) when their waves cost no more than the 128 x 256
// tiles' waves, which picks the faster of the two at every T measured
// (640 ... 8192 rows, width 6144: small below 1024 and for 1536 ... 3072).
// The down product always takes them and splits its reduction to fill the
// CUs (see tiled_dense_splits).
constexpr int kDenseCus = 256;
bool dense_gu_big(int T, int Is)
{
    const long long n = Is / 128;  // 128-channel gate + up column tiles
    const long long big = (T + 255) / 256 * n, small = (T + 127) / 128 * n;
    return 2 * ((big + kDenseCus - 1) / kDenseCus) <= (small + kDenseCus - 1) / kDenseCus;
}
int gu_cfg(int T, int K, int E, int Is)
{
    if (K == 0) return Is % 128 == 0 && dense_gu_big(T, Is) ? 3 : kTlGuWide;
    return (long long)T * K <= (long long)kTlMidGuRows * E ? kTlMid : kTlGuWide;
}
int dn_cfg(int T, int K, int E)
{
    if (K == 0) return 3;
    if ((long long)T * K <= (long long)kTlMidDnRows * E) return kTlMid;
    return big_batch(T, K, E) ? kTlDnBig : kTlDnSmall;
}
// the 16-row tiles of a MoE layer and the 32-row tiles of a dense layer.
// The down product leaves the 16-row tiles from kMidDnFromT tokens on where it
// takes the 64-row ones (T K <= kTlMidDnRows E): Flint shape T = 448 down
// 119.5 -> 113.6 us, 512 123.1 -> 116.6 (no change at 384; gate/up on 64-row
// tiles no faster there: 205 -> 208 us at 448).
constexpr int kMidDnFromT = 448;
bool moe_small_tiles(int T, int K) { return K > 0 && T < kLargeTilesFromT; }
bool moe_small_down(int T, int K, int E)
{
    return moe_small_tiles(T, K) && (T < kMidDnFromT || dn_cfg(T, K, E) != kTlMid);
}
bool dense_small_tiles(int T, int K) { return K == 0 && T < kDenseTiledFromT; }

template <int MODE, typename C>
hipError_t launch_cfg(TiledArgs ta, hipStream_t stream, Marks m)
{
    const ExpertArgs &a = ta.e;
    const int mt = (a.T + C::BM - 1) / C::BM;
    int items;
    if (MODE == ROUTER) {
        items = mt * ((a.E + C::BN - 1) / C::BN) * ta.ksplit;
    } else {
        const int ntn_s = MODE == GATE_UP ? a.Is / (C::BN / 2) : (a.H + C::BN - 1) / C::BN;
        const int ntn_r = MODE == GATE_UP ? a.I / (C::BN / 2) : (a.H + C::BN - 1) / C::BN;
        ta.n_shared = a.Is > 0 ? mt * ntn_s * (MODE == DOWN && a.shared_splits > 1 ? a.shared_splits : 1) : 0;
        items = (ta.n_shared + kXcds - 1) / kXcds * kXcds + list_capacity(a.T, a.K, a.E, C::BM) * ntn_r;
    }
    const int grid = (items + kXcds - 1) / kXcds * kXcds;
    return launch_k(k_tiled<MODE, C>, grid, C::THREADS, 0, stream, m, ta);
}

template <int MODE>
hipError_t launch_mode(int which, const TiledArgs &ta, hipStream_t stream, Marks m)
{
    switch (which) {
    case 1: return launch_cfg<MODE, CfgWide>(ta, stream, m);
    case 2: return launch_cfg<MODE, CfgBig>(ta, stream, m);
    case 3: return launch_cfg<MODE, CfgBig8>(ta, stream, m);
    case 6:
        // 128 x 256 tiles (128 gate + 128 up channels): whole tiles of the widths, else 128 x 128
        if (MODE != GATE_UP || (ta.e.I % 128 == 0 && ta.e.Is % 128 == 0)) return launch_cfg<MODE, CfgWideN>(ta, stream, m);
        return launch_cfg<MODE, CfgSmall>(ta, stream, m);
    case kTlMid:
        // 64 x 256 tiles (128 gate + 128 up channels): whole tiles of the widths, else 64 x 128
        if constexpr (MODE == GATE_UP)
            if (ta.e.I % 128 != 0 || ta.e.Is % 128 != 0) return launch_cfg<MODE, CfgMidN>(ta, stream, m);
        return launch_cfg<MODE, CfgMid>(ta, stream, m);
    default: return launch_cfg<MODE, CfgSmall>(ta, stream, m);
    }
}

}  // namespace

bool tiled_eligible(int T, int K, int E, int H, int I, int Is, bool bf16)
{
    // whole k slices (H, I, Is); a gate/up tile takes BN/2 gate channels and
    // the same up channels
    const int which = gu_cfg(T, K, E, Is);
    const int half = cfg_bn(which == 6 || which == kTlMid ? 0 : which) / 2;  // CfgWideN, CfgMid fall back to 128-column tiles
    return bf16 && H % 64 == 0 && I % 64 == 0 && Is % 64 == 0 && I % half == 0 && Is % half == 0;
}

// The dense down product on 256 x 256 tiles reduces over the whole width,
// with few tiles for moderate T (T = 4096, H = 2048: 128 tiles on 256 CUs).
// It is split into the most partial arrays (a power of two up to 8, each a
// whole number of 64-wide slices) that keep the items within one wave; the
// combine adds them.  Measured (H = 2048, width 6144, layer time): T = 640
// 112 -> 85 us (8 splits), 2048 225 -> 202 (4), 3072 347 -> 293 (2), 4096
// 349 -> 342 (2); at 8192 one split (256 tiles) is best.
int tiled_dense_splits(int T, int H, int Is)
{
    if (dense_small_tiles(T, 0)) {
        // 32-row tiles of 64 columns: H/64 per row tile, too few to fill the CUs
        // alone; the most splits up to 8 whose slices stay whole (T = 32, width
        // 6144: 8 splits, 256 items)
        int best = 1;
        for (int s = 2; s <= 8; ++s)
            if (Is % (CfgDecDn::BK * s) == 0) best = s;
        return best;
    }
    const long long tiles = (long long)(T + 255) / 256 * ((H + 255) / 256);
    int s = 1;
    while (s < 8 && tiles * (2 * s) <= kDenseCus && Is % (64 * 2 * s) == 0) s *= 2;
    return s;
}

int tiled_bm1(int T, int K, int E, int Is)
{
    if (moe_small_tiles(T, K)) return CfgMoeGu::BM;
    if (dense_small_tiles(T, K)) return CfgDecGu::BM;
    return cfg_bm(gu_cfg(T, K, E, Is));
}
int tiled_bm2(int T, int K, int E)
{
    if (moe_small_down(T, K, E)) return CfgMoeDn::BM;
    if (dense_small_tiles(T, K)) return CfgDecDn::BM;
    return cfg_bm(dn_cfg(T, K, E));
}

hipError_t launch_experts_tiled(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    TiledArgs ta{};
    ta.e = a;
    if (moe_small_tiles(a.T, a.K)) {
        const hipError_t err = launch_cfg<GATE_UP, CfgMoeGu>(ta, stream, marks ? marks[0] : Marks{});
        if (err != hipSuccess) return err;
        const Marks m = marks ? marks[1] : Marks{};
        return moe_small_down(a.T, a.K, a.E) ? launch_cfg<DOWN, CfgMoeDn>(ta, stream, m)
                                              : launch_mode<DOWN>(dn_cfg(a.T, a.K, a.E), ta, stream, m);
    }
    if (dense_small_tiles(a.T, a.K)) {
        // a dense layer at decode sizes (layer times measured on the dense layer,
        // H = 2048, width 6144, against the weight-streaming kernels: T = 1
        // 27.6 -> 25.4 us, T = 32 35.2 -> 28.6, T = 64 50.6 -> 35.6, T = 128
        // 73.5 -> 48.6)
        const Marks m = marks ? marks[0] : Marks{};
        const hipError_t err = a.T <= kDecGuRows6 ? launch_cfg<GATE_UP, CfgDecGu>(ta, stream, m)
                                                  : launch_cfg<GATE_UP, CfgDecGu4>(ta, stream, m);
        if (err != hipSuccess) return err;
        return launch_cfg<DOWN, CfgDecDn>(ta, stream, marks ? marks[1] : Marks{});
    }
    const hipError_t err = launch_mode<GATE_UP>(gu_cfg(a.T, a.K, a.E, a.Is), ta, stream, marks ? marks[0] : Marks{});
    if (err != hipSuccess) return err;
    return launch_mode<DOWN>(dn_cfg(a.T, a.K, a.E), ta, stream, marks ? marks[1] : Marks{});
}

bool tiled_router_eligible(int T, int H, bool bf16) { return bf16 && T >= 1024 && H % (64 * kRouterSplits) == 0; }

// Split the sum over H while the batch alone gives too few tiles to fill the
// chip (measured: faster up to 4096 tokens; at 16384 the extra partial
// arrays cost more than they save).
int router_splits(int T, int H, int E, bool bf16)
{
    if (T < 1024) return small_router_splits(T, H, E);
    return tiled_router_eligible(T, H, bf16) && T <= 4096 ? kRouterSplits : 1;
}

hipError_t launch_router_tiled(const void *x, int T, int H, const void *router, const float *bias, int E,
                               float *logits, hipStream_t stream, Marks m)
{
    TiledArgs ta{};
    ta.e.x = x;
    ta.e.T = T;
    ta.e.H = H;
    ta.e.E = E;
    ta.router = router;
    ta.bias = bias;
    ta.logits = logits;
    ta.ksplit = router_splits(T, H, E, true);
    return launch_cfg<ROUTER, CfgRouter>(ta, stream, m);
}

}  // namespace flint
