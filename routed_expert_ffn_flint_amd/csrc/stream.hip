// Persistent weight-streaming expert kernels for small batches (decode).
//
// Layer (serving-kit review, "The architecture, from the config"; release news
// page, "What runs on each token"): K selected experts of width I per token plus
// an always-on shared expert of width Is, each a gated three-matrix SwiGLU.
//
// At decode batch sizes every selected expert holds a handful of rows, so the
// layer is a stream of expert weights from HBM; the kernels here are built to
// keep that stream full:
//   - a fixed grid of work-groups (a few per CU) walks the work items with a
//     static stride, so per-group setup is paid once, not per tile;
//   - each work-group first copies the dispatch tables (tile list, expert
//     offsets, and for gate/up the expert-sorted token list) into LDS, so
//     setting up an item costs LDS reads only and never waits on the
//     vector-memory counter, which would also wait for the weights in flight;
//   - each wave streams its quarter of the reduction dimension in batches of U
//     32-wide slices, the next batch (of this item or of the next one) issued
//     before the current batch's MFMAs, so weight loads stay in flight across
//     item boundaries;
//   - the four waves' partial sums are added in LDS in wave order (the result
//     does not depend on timing).
// Gate/up items: MB*16 rows x (NB/2)*16 channels of gate and of up, SwiGLU
// fused (16 x 16 + 16 for batches of up to 64 tokens, else 32 x 32 + 32).
// Down items: 32 rows x NB*16 output columns.
#include "gemm_core.hpp"
#include "launch.hpp"

constexpr int kStNb1 = 4;  // gate/up items: NB1/2 blocks of 16 channels
constexpr int kStNb2 = 2;  // down items: NB2 blocks of 16 columns
constexpr int kStUmax1 = 2;  // gate/up slices per batch (register budget: 2 batches in flight)
constexpr int kStUmax2 = 2;  // down slices per batch
constexpr int kStMb1 = 2;  // gate/up items: MB1 blocks of 16 rows
// Batches of at most kStSmallT tokens (an expert then gets a row or
// two) use gate/up items of kStMb1s row blocks x kStNb1s column
// blocks: half the activation loads, and twice the items, which evens out the
// last round of the persistent grid (measured 108 -> 103 us at T = 32; at
// T = 256 the larger items are faster).
constexpr int kStSmallT = 64;
constexpr int kStMb1s = 1;
constexpr int kStNb1s = 2;
constexpr int kStWgs1 = 2;  // gate/up: work-groups per CU (the grid; also the occupancy asked for)
constexpr int kStWgs2 = 2;  // down

constexpr int kStMb2 = 2;  // down items: MB2 blocks of 16 rows

namespace flint {

namespace {

constexpr int kWaves = 4;

// Dispatch tables in the kernel's dynamic LDS: the tile list's (expert,
// first slot) pairs at [0, 2 nlist), the expert offsets (E + 1) after them, and
// for gate/up the token of each slot (T K) after those.  The kernel indexes
// the LDS array itself, never a pointer into it: read through a pointer kept
// in a struct, the offsets had become flat loads, and the wait of a flat load
// (like that of a global load of the token list) also waits for every weight
// load in flight, so each item's setup drained the stream.
struct TableLayout {
    int nlist, offsets, tokens;  // list length; word index of the offsets and of the tokens
};

__device__ __forceinline__ TableLayout load_tables(const ExpertArgs &a, const int32_t *glist, int nlist,
                                                   bool tokens, int32_t *lds)
{
    TableLayout t{nlist, 2 * nlist, 2 * nlist + a.E + 1};
    // the three arrays as one range of words (a dense layer, K = 0, has shared
    // items only and no dispatch tables), each thread's loads all issued
    // before the first is waited for
    const int n_off = a.K > 0 ? a.E + 1 : 0;
    const int total = t.offsets + n_off + (tokens && a.K > 0 ? a.T * a.K : 0);
    constexpr int kPer = 4;
    for (int i0 = threadIdx.x; i0 < total; i0 += kPer * blockDim.x) {
        int v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = min(i0 + u * (int)blockDim.x, total - 1);
            const int32_t *src = i < t.offsets ? glist + i
                                 : i < t.tokens ? a.offsets + (i - t.offsets)
                                                : a.sorted_token + (i - t.tokens);
            v[u] = *src;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = i0 + u * (int)blockDim.x;
            if (i < total) lds[i] = v[u];
        }
    }
    __syncthreads();
    return t;
}

// What one wave needs for one work item.
template <typename S, int MB, int NB>
struct Item {
    const S *a[MB];
    const S *b[NB];
    int s0;          // first slice of this wave
    int nbatch;      // batches of U slices for this wave
    int row0, row_end, n0, kdim;
    int ysplit;      // shared down items: which partial array of y_shared
    int shared;      // 1: shared-expert item
    int valid;
};

}  // namespace

// GATE_UP: gate/up + SwiGLU -> h (dtype);  otherwise: down -> y (float32).
template <typename DT, int MB, int NB, int U, bool GATE_UP>
__global__ __launch_bounds__(256, GATE_UP ? kStWgs1 : kStWgs2) void k_expert_stream(ExpertArgs a,
                                                                                          int n_shared_items)
{
    using S = typename DT::storage;
    constexpr int BM = MB * 16;
    constexpr int HALF = NB / 2;
    constexpr int BN = GATE_UP ? HALF * 16 : NB * 16;  // channels (gate/up) or columns (down) per item
    extern __shared__ int32_t dyn_lds[];
    __shared__ float red[kWaves * MB * NB * 256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = (lane >> 4) * 8;
    const int H = a.H;
    const int nlist = GATE_UP ? (a.K > 0 ? a.meta[0] : 0) : (a.K > 0 ? a.meta[1] : 0);
    const TableLayout tab = load_tables(a, GATE_UP ? a.list1 : a.list2, nlist, GATE_UP, dyn_lds);

    const int ntn_shared = GATE_UP ? a.Is / BN : (H + BN - 1) / BN;
    const int ntn_routed = GATE_UP ? a.I / BN : (H + BN - 1) / BN;
    const int n_items = n_shared_items + nlist * ntn_routed;

    auto get = [&](int item) {
        Item<S, MB, NB> it;
        it.valid = item < n_items;
        if (!it.valid) item = 0;  // a valid item's addresses, used only as dummy prefetch targets
        int e = 0, nt;
        int klen, kfirst = 0;  // this item's reduction: slices [kfirst, kfirst + klen/32)
        const S *wa, *wb;  // gate/up (GATE_UP) or the down matrix (wa)
        it.ysplit = 0;
        if (item < n_shared_items) {
            // shared down items come in shared_splits parts of the reduction
            const int nsplit = GATE_UP ? 1 : (a.shared_splits > 1 ? a.shared_splits : 1);
            const int sh = item / nsplit;
            it.ysplit = item % nsplit;
            it.shared = 1;
            it.row0 = (sh / ntn_shared) * BM;
            nt = sh % ntn_shared;
            it.row_end = a.T;
            it.kdim = GATE_UP ? H : a.Is;
            klen = it.kdim / nsplit;
            kfirst = it.ysplit * (klen / 32);
            wa = GATE_UP ? (const S *)a.shared_gate : (const S *)a.shared_down;
            wb = (const S *)a.shared_up;
        } else {
            it.shared = 0;
            const int r = item - n_shared_items;
            const int entry = r / ntn_routed;
            nt = r % ntn_routed;
            e = dyn_lds[2 * entry];
            it.row0 = dyn_lds[2 * entry + 1];
            it.row_end = dyn_lds[tab.offsets + e + 1];
            it.kdim = GATE_UP ? H : a.I;
            klen = it.kdim;
            wa = GATE_UP ? (const S *)a.gate + (size_t)e * a.I * H : (const S *)a.down + (size_t)e * H * a.I;
            wb = GATE_UP ? (const S *)a.up + (size_t)e * a.I * H : nullptr;
        }
        it.n0 = nt * BN;
        const int per = klen / 32 / kWaves;  // slices per wave (the launcher checks divisibility)
        it.s0 = kfirst + wave * per;
        it.nbatch = per / U;
        if (GATE_UP) {
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                const int c = it.n0 + j * 16 + (lane & 15);
                it.b[j] = wa + (size_t)c * H + kg;
                it.b[j + HALF] = wb + (size_t)c * H + kg;
            }
        } else {
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                int c = it.n0 + n * 16 + (lane & 15);
                if (c >= H) c = 0;
                it.b[n] = wa + (size_t)c * it.kdim + kg;
            }
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            int r = it.row0 + m * 16 + (lane & 15);
            if (r >= it.row_end) r = it.row0;  // rows past the tile repeat its first row (cache hits)
            if (GATE_UP) {
                const int tok = it.shared ? r : dyn_lds[tab.tokens + r];
                it.a[m] = (const S *)a.x + (size_t)tok * H + kg;
            } else {
                it.a[m] = (it.shared ? (const S *)a.h_shared : (const S *)a.h_sorted) + (size_t)r * it.kdim + kg;
            }
        }
        return it;
    };

    auto load_batch = [&](const Item<S, MB, NB> &it, int batch, Frag<DT> (&fb)[U][NB], Frag<DT> (&fa)[U][MB]) {
        const int s = it.s0 + batch * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int n = 0; n < NB; ++n) fb[u][n].load(it.b[n] + (s + u) * 32);
#pragma unroll
            for (int m = 0; m < MB; ++m) fa[u][m].load(it.a[m] + (s + u) * 32);
        }
    };

    // Two register buffers in ping-pong: while one batch is multiplied, the
    // other batch's loads are in flight (each item has an even number of
    // batches per wave, so item i's last batch always sits in buffer B and
    // the next item's first batch goes to buffer A).
    int item = blockIdx.x;
    Item<S, MB, NB> cur = get(item);
    if (!cur.valid) return;  // uniform across the work-group
    Frag<DT> ab[U][NB], aa[U][MB], bb[U][NB], ba[U][MB];
    load_batch(cur, 0, ab, aa);
    while (true) {
        const Item<S, MB, NB> nxt = get(item + gridDim.x);
        f32x4 acc[MB][NB];
        zero_acc(acc);
        for (int j = 0; j < cur.nbatch; j += 2) {
            // scheduling barriers keep each phase in program order, so that a
            // buffer's loads are issued before the other buffer's MFMAs wait
            load_batch(cur, j + 1, bb, ba);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int n = 0; n < NB; ++n) mma(acc[m][n], aa[u][m], ab[u][n]);
            // buffer A: this item's batch j+2, else the next item's first batch
            // (a dummy reload when there is no next item keeps the count of
            // loads in flight fixed)
            const bool more = j + 2 < cur.nbatch;
            __builtin_amdgcn_sched_barrier(0);
            load_batch(more ? cur : nxt, more ? j + 2 : 0, ab, aa);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int n = 0; n < NB; ++n) mma(acc[m][n], ba[u][m], bb[u][n]);
            __builtin_amdgcn_sched_barrier(0);
        }
        splitk_reduce<kWaves, MB, NB>(acc, red);
        if (GATE_UP) {
            S *hout = cur.shared ? (S *)a.h_shared : (S *)a.h_sorted;
            const int width = cur.shared ? a.Is : a.I;
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                if ((j % kWaves) != wave) continue;
                const int c = cur.n0 + j * 16 + (lane & 15);
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = cur.row0 + m * 16 + (lane >> 4) * 4 + i;
                        if (r < cur.row_end)
                            store_elem<DT>(hout + (size_t)r * width + c, swiglu(acc[m][j][i], acc[m][j + HALF][i]));
                    }
            }
        } else {
            float *yout = cur.shared ? a.y_shared + (size_t)cur.ysplit * a.T * H : a.y_sorted;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                if ((n % kWaves) != wave) continue;
                const int c = cur.n0 + n * 16 + (lane & 15);
                if (c >= H) continue;
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = cur.row0 + m * 16 + (lane >> 4) * 4 + i;
                        if (r < cur.row_end) yout[(size_t)r * H + c] = acc[m][n][i];
                    }
            }
        }
        __syncthreads();  // every wave has read `red` before the next item overwrites it
        if (!nxt.valid) break;
        cur = nxt;
        item += gridDim.x;
    }
}

// Eligible shapes: every item's reduction dimension splits evenly into 4 waves
// x an even number of batches of U slices (gate/up: H; down: I and Is).
static int unroll_for(const int *dims, int n, int umax)
{
    for (int U : {4, 2, 1}) {
        if (U > umax) continue;
        bool ok = true;
        for (int i = 0; i < n; ++i) ok = ok && dims[i] % (32 * kWaves * U * 2) == 0;
        if (ok) return U;
    }
    return 0;
}
static int unroll_gate_up(int H) { return unroll_for(&H, 1, kStUmax1); }
static int unroll_down(int I, int Is)
{
    const int d[2] = {I, Is > 0 ? Is : I};
    return unroll_for(d, 2, kStUmax2);
}

bool stream_eligible(int T, int H, int I, int Is)
{
    return T <= kStreamMaxT && unroll_gate_up(H) > 0 && unroll_down(I, Is) > 0;
}
// (routed layers only: a dense layer's gate/up items are all shared-expert
// items, and there the 32 x 64 items measured faster at T = 32, 18 vs 22 us)
static bool small_batch(int T, int K) { return T <= kStSmallT && K > 0; }
int stream_bm1(int T, int K) { return (small_batch(T, K) ? kStMb1s : kStMb1) * 16; }
int stream_bm2() { return kStMb2 * 16; }

template <typename DT, int U, bool GATE_UP>
static hipError_t launch_one(const ExpertArgs &a, int grid, int n_shared, size_t lds, hipStream_t stream, Marks m)
{
    if (GATE_UP && small_batch(a.T, a.K))
        return launch_k(k_expert_stream<DT, kStMb1s, kStNb1s, U, true>, grid, 256, lds, stream, m, a,
                        n_shared);
    if (GATE_UP)
        return launch_k(k_expert_stream<DT, kStMb1, kStNb1, U, true>, grid, 256, lds, stream, m, a,
                        n_shared);
    return launch_k(k_expert_stream<DT, kStMb2, kStNb2, U, false>, grid, 256, lds, stream, m, a, n_shared);
}

template <typename DT, bool GATE_UP>
static hipError_t launch_u(int U, const ExpertArgs &a, int grid, int n_shared, size_t lds, hipStream_t stream,
                           Marks m)
{
    if (U == 4) return launch_one<DT, 4, GATE_UP>(a, grid, n_shared, lds, stream, m);
    if (U == 2) return launch_one<DT, 2, GATE_UP>(a, grid, n_shared, lds, stream, m);
    return launch_one<DT, 1, GATE_UP>(a, grid, n_shared, lds, stream, m);
}

template <typename DT>
static hipError_t launch_stream_t(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    const int bm1 = stream_bm1(a.T, a.K), bm2 = kStMb2 * 16;
    const int bn1 = (small_batch(a.T, a.K) ? kStNb1s : kStNb1) / 2 * 16, bn2 = kStNb2 * 16;
    const int cap1 = list_capacity(a.T, a.K, a.E, bm1);
    const int cap2 = list_capacity(a.T, a.K, a.E, bm2);
    const int ns1 = a.Is > 0 ? (a.T + bm1 - 1) / bm1 * (a.Is / bn1) : 0;
    const int nsplit = a.shared_splits > 1 ? a.shared_splits : 1;
    const int ns2 = a.Is > 0 ? (a.T + bm2 - 1) / bm2 * ((a.H + bn2 - 1) / bn2) * nsplit : 0;
    const int max1 = ns1 + cap1 * (a.I / bn1);
    const int max2 = ns2 + cap2 * ((a.H + bn2 - 1) / bn2);
    const size_t lds1 = (size_t)(2 * cap1 + a.E + 1 + (a.K > 0 ? a.T * a.K : 0)) * 4;
    const size_t lds2 = (size_t)(2 * cap2 + a.E + 1) * 4;
    const hipError_t err = launch_u<DT, true>(unroll_gate_up(a.H), a, min(kStWgs1 * a.cus, max1), ns1, lds1, stream,
                                              marks ? marks[0] : Marks{});
    if (err != hipSuccess) return err;
    return launch_u<DT, false>(unroll_down(a.I, a.Is / nsplit), a, min(kStWgs2 * a.cus, max2), ns2, lds2, stream,
                               marks ? marks[1] : Marks{});
}

hipError_t launch_experts_stream(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    return a.bf16 ? launch_stream_t<BF16>(a, stream, marks) : launch_stream_t<F32>(a, stream, marks);
}

}  // namespace flint
