// Persistent weight-streaming expert kernels for block-scaled 4-bit expert
// weights (MXFP4), small batches.
//
// Layer (serving-kit review, "The architecture, from the config"; release news
// page, "What runs on each token"): K selected experts of width I per token plus
// an always-on shared expert of width Is, each a gated three-matrix SwiGLU.
// Weight format (a definition; the pages' low-bit builds store 4-bit weights,
// "Recursive launches Flint: open-weight coding model with 39.8 billion
// parameters for local execution", section "What Flint is, and how it is
// built"): OCP Microscaling MXFP4 -- FP4 E2M1 elements,
// 32-element blocks along the reduction dimension, an E8M0 scale 2^(s-127) per
// block, two elements per byte with the lower-indexed one in the low nibble --
// stored in tiles of 16 rows x one block: a tile's codes are its 16 rows' 16
// bytes back to back (256 B), its scales 16 bytes; tiles run along the
// reduction dimension, then down the rows.
//
// Same structure as the bf16 streaming kernels (persistent grid, tile list in
// LDS, ping-pong register buffers; gate/up items shared by four waves that
// split the reduction dimension and add their partial sums in wave order),
// except that a down item (a reduction of only I) belongs to one wave, which
// needs neither LDS sums nor barriers; the weight side is 4-bit:
//   - a step covers CK values of k per wave; lane l = row + 16*g takes
//     elements [k0 + g*CK/4, +CK/4) of its row, which lie in one block: CK/8
//     code bytes and one scale byte per weight row.  With the tiled storage
//     the 64 lanes' code bytes are one contiguous stretch (1 KB for CK=128) and
//     their scale bytes another, so every load is fully coalesced (row-major
//     storage puts each lane on another row and costs the address unit about
//     four times as many cache accesses per load);
//   - the activations use the same assignment of k to lanes, so MFMA j of the
//     step multiplies elements k0 + g*CK/4 + 8j .. +7 on both sides (the k
//     order of the sum is permuted, its value is not);
//   - v_cvt_scalef32_pk_bf16_fp4 turns two codes into two bf16 values times
//     the block scale, exactly (E2M1 x 2^n is a bf16 value), so the MFMAs are
//     the bf16 ones and everything after them is as in the bf16 path.
#include "gemm_core.hpp"
#include "launch.hpp"

constexpr int kMxWgs = 2;  // work-groups per CU (grid and occupancy)

namespace flint {

namespace {

constexpr int kWavesMx = 4;

// E8M0 scale byte -> float (2^(s-127); 0 is the denormal 2^-127, 255 NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return __uint_as_float(s == 0 ? 0x00400000u : (s == 255 ? 0x7fc00000u : s << 23));
}

// 8 codes (one dword) times the scale -> one bf16 fragment (8 values, in order).
__device__ __forceinline__ void fp4x8_to_frag(uint32_t codes, float sc, Frag<BF16> &f)
{
    u32x4 u;
    u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
    u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
    u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
    u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
    f.v = __builtin_bit_cast(bf16x8, u);
}

// Codes of one step for one weight row: CK/8 bytes (8 or 16).
template <int CK> struct CodeVec {
    static constexpr int W = CK / 32;  // dwords
    uint32_t w[W];
    __device__ __forceinline__ void load(const uint8_t *p)
    {
        if constexpr (W == 2) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            w[0] = v.x;
            w[1] = v.y;
        } else {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
            w[0] = v[0];
            w[1] = v[1];
            w[2] = v[2];
            w[3] = v[3];
        }
    }
};

// What one wave needs for one work item.  Pointers and strides are the same
// for every lane (kept in scalar registers); each lane adds its own 32-bit
// offset, so an item costs a few vector registers whatever NB is.
template <int MB>
struct MxItem {
    const uint8_t *qa, *qb;  // codes of the tile row holding row n0: gate (or down), up
    const uint8_t *sa, *sb;  // scales likewise
    const uint16_t *abase;   // activations (x, h_sorted or h_shared)
    uint32_t qrow, srow;     // bytes per tile row (16 weight rows): codes, scales
    uint32_t qoff, soff;     // this lane's row (lane & 15) and first k within a tile row, in bytes
    uint32_t aoff[MB];       // this lane's activation row and first k, in elements
    int nstep;               // steps of this wave
    int row0, row_end, n0, shared, valid;
};

}  // namespace

// GATE_UP: gate/up + SwiGLU -> h (bf16);  otherwise: down -> y (float32).
// MB row blocks of 16, NB column blocks of 16 (gate/up: NB/2 gate + NB/2 up).
// KSPLIT 4: the four waves of a work-group share each item, a quarter of the
// reduction each, and add their partial sums in LDS; KSPLIT 1: every wave
// walks its own items over the whole reduction (no LDS sums, no barriers).
template <int MB, int NB, int CK, bool GATE_UP, int KSPLIT>
__global__ __launch_bounds__(256, kMxWgs) void k_expert_stream_mx4(ExpertArgs a, int n_shared_items)
{
    constexpr int BM = MB * 16;
    constexpr int HALF = NB / 2;
    constexpr int BN = GATE_UP ? HALF * 16 : NB * 16;
    constexpr int NF = CK / 32;  // fragments (MFMA k-steps) per step
    static_assert(CK == 64 || CK == 128, "a lane's slice (CK/4 elements) lies in one 32-element block");
    extern __shared__ int32_t dyn_lds[];
    static_assert(KSPLIT == 1 || KSPLIT == kWavesMx, "waves per item");
    __shared__ float red[KSPLIT > 1 ? kWavesMx * MB * NB * 256 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int H = a.H;
    const int nlist = GATE_UP ? a.meta[0] : a.meta[1];
    int32_t *list = dyn_lds;
    int32_t *offsets = dyn_lds + 2 * nlist;
    int32_t *toks = offsets + a.E + 1;  // expert-sorted token list (gate/up)
    for (int i = threadIdx.x; i < 2 * nlist; i += blockDim.x) list[i] = (GATE_UP ? a.list1 : a.list2)[i];
    for (int i = threadIdx.x; i <= a.E; i += blockDim.x) offsets[i] = a.offsets[i];
    if (GATE_UP)
        for (int i = threadIdx.x; i < a.T * a.K; i += blockDim.x) toks[i] = a.sorted_token[i];
    __syncthreads();

    const int ntn_shared = GATE_UP ? a.Is / BN : H / BN;
    const int ntn_routed = GATE_UP ? a.I / BN : H / BN;
    const int n_items = n_shared_items + nlist * ntn_routed;

    auto get = [&](int item) {
        MxItem<MB> it;
        it.valid = item < n_items;
        if (!it.valid) item = 0;  // a valid item's addresses, used only as dummy prefetch targets
        int nt, kdim, wrows;
        if (item < n_shared_items) {
            it.shared = 1;
            it.row0 = (item / ntn_shared) * BM;
            nt = item % ntn_shared;
            it.row_end = a.T;
            kdim = GATE_UP ? H : a.Is;
            wrows = 0;
            it.qa = (const uint8_t *)(GATE_UP ? a.shared_gate : a.shared_down);
            it.sa = GATE_UP ? a.shared_gate_s : a.shared_down_s;
            it.qb = (const uint8_t *)a.shared_up;
            it.sb = a.shared_up_s;
        } else {
            it.shared = 0;
            const int r = item - n_shared_items;
            const int entry = r / ntn_routed;
            nt = r % ntn_routed;
            // list entries and offsets are the same in every lane
            const int e = __builtin_amdgcn_readfirstlane(list[2 * entry]);
            it.row0 = __builtin_amdgcn_readfirstlane(list[2 * entry + 1]);
            it.row_end = __builtin_amdgcn_readfirstlane(offsets[e + 1]);
            kdim = GATE_UP ? H : a.I;
            wrows = e * (GATE_UP ? a.I : H);  // weight rows of earlier experts
            it.qa = (const uint8_t *)(GATE_UP ? a.gate : a.down);
            it.sa = GATE_UP ? a.gate_s : a.down_s;
            it.qb = (const uint8_t *)a.up;
            it.sb = a.up_s;
        }
        it.n0 = nt * BN;
        it.qrow = kdim * 8;   // kdim/32 tiles of 256 code bytes
        it.srow = kdim / 2;   // kdim/32 tiles of 16 scale bytes
        const size_t first_tile_row = ((size_t)wrows + it.n0) / 16;
        it.qa += first_tile_row * it.qrow;
        it.qb += first_tile_row * it.qrow;
        it.sa += first_tile_row * it.srow;
        it.sb += first_tile_row * it.srow;
        it.nstep = kdim / CK / KSPLIT;  // the launcher checks divisibility (and evenness)
        const int kw = (KSPLIT > 1 ? wave * it.nstep * CK : 0) + g * (CK / 4);  // this lane's first k
        // tile kw/32, the lane's row within it, the byte of element kw in that row
        it.qoff = (kw / 32) * 256 + (lane & 15) * 16 + (kw % 32) / 2;
        it.soff = (kw / 32) * 16 + (lane & 15);
        it.abase = GATE_UP ? (const uint16_t *)a.x
                           : (it.shared ? (const uint16_t *)a.h_shared : (const uint16_t *)a.h_sorted);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            int r = it.row0 + m * 16 + (lane & 15);
            if (r >= it.row_end) r = it.row0;  // rows past the tile repeat its first row (cache hits)
            const int arow = GATE_UP ? (it.shared ? r : toks[r]) : r;
            it.aoff[m] = (uint32_t)arow * (GATE_UP ? H : kdim) + kw;
        }
        return it;
    };

    // raw step buffers: activation fragments, weight codes, scale bytes
    struct Raw {
        Frag<BF16> fa[MB][NF];
        CodeVec<CK> q[NB];
        uint32_t s[NB];
    };
    auto load = [&](const MxItem<MB> &it, int step, Raw &r) {
        // a step advances CK/32 tiles; with lane l = row + 16 * group, the lanes
        // of one load read one contiguous stretch of codes (CK * 8 bytes)
        const uint32_t qo = it.qoff + step * (CK * 8), so = it.soff + step * (CK / 2);
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const bool up = GATE_UP && n >= HALF;
            const uint32_t trow = (uint32_t)(GATE_UP ? n % HALF : n);  // tile rows past the first
            r.q[n].load((up ? it.qb : it.qa) + trow * it.qrow + qo);
            r.s[n] = (up ? it.sb : it.sa)[trow * it.srow + so];
        }
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < NF; ++j) r.fa[m][j].load(it.abase + (it.aoff[m] + step * CK + 8 * j));
    };
    f32x4 acc[MB][NB];
    auto compute = [&](const Raw &r) {
        float sc[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            // the empty asm pins the scale decode here: without it the compiler
            // hoists the decode's compares to just after the scale load is
            // issued, and the wave then waits on that load a phase early
            uint32_t sv = r.s[n];
            asm volatile("" : "+v"(sv));
            sc[n] = e8m0_to_f32(sv);
        }
        // k-slice outer, columns inner: consecutive MFMAs use different
        // accumulators, so none waits for the previous one's result
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                Frag<BF16> fb;
                fp4x8_to_frag(r.q[n].w[j], sc[n], fb);
#pragma unroll
                for (int m = 0; m < MB; ++m) mma(acc[m][n], r.fa[m][j], fb);
            }
    };

    // KSPLIT 4: work-group b takes items b, b + grid, ...; KSPLIT 1: wave w of
    // work-group b takes items 4b + w, 4b + w + 4 grid, ...
    int item = KSPLIT > 1 ? blockIdx.x : blockIdx.x * kWavesMx + wave;
    const int stride = KSPLIT > 1 ? gridDim.x : gridDim.x * kWavesMx;
    MxItem<MB> cur = get(item);
    if (!cur.valid) return;  // uniform across the work-group (KSPLIT 4) or the wave (1)
    Raw ra, rb;
    load(cur, 0, ra);
    while (true) {
        const MxItem<MB> nxt = get(item + stride);
        zero_acc(acc);
        for (int st = 0; st < cur.nstep; st += 2) {
            // scheduling barriers keep each phase in program order, so that a
            // buffer's loads are issued before the other buffer is consumed
            load(cur, st + 1, rb);
            __builtin_amdgcn_sched_barrier(0);
            compute(ra);
            // buffer A: this item's step st+2, else the next item's first step
            // (a dummy reload when there is no next item keeps the count of
            // loads in flight fixed)
            const bool more = st + 2 < cur.nstep;
            __builtin_amdgcn_sched_barrier(0);
            load(more ? cur : nxt, more ? st + 2 : 0, ra);
            __builtin_amdgcn_sched_barrier(0);
            compute(rb);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (KSPLIT > 1) splitk_reduce<kWavesMx, MB, NB>(acc, red);
        if (GATE_UP) {
            uint16_t *hout = cur.shared ? (uint16_t *)a.h_shared : (uint16_t *)a.h_sorted;
            const int width = cur.shared ? a.Is : a.I;
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                if (KSPLIT > 1 && (j % kWavesMx) != wave) continue;
                const int c = cur.n0 + j * 16 + (lane & 15);
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = cur.row0 + m * 16 + (lane >> 4) * 4 + i;
                        if (r < cur.row_end)
                            hout[(size_t)r * width + c] = f32_to_bf16(swiglu(acc[m][j][i], acc[m][j + HALF][i]));
                    }
            }
        } else {
            float *yout = cur.shared ? a.y_shared : a.y_sorted;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                if (KSPLIT > 1 && (n % kWavesMx) != wave) continue;
                const int c = cur.n0 + n * 16 + (lane & 15);
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = cur.row0 + m * 16 + (lane >> 4) * 4 + i;
                        if (r < cur.row_end) yout[(size_t)r * H + c] = acc[m][n][i];
                    }
            }
        }
        if (KSPLIT > 1) __syncthreads();  // every wave has read `red` before the next item overwrites it
        if (!nxt.valid) break;
        cur = nxt;
        item += stride;
    }
}

namespace {
// gate/up (1) and down (2) items: MB blocks of 16 rows; NB blocks of 16
// columns (gate/up: NB/2 blocks of gate and of up channels); CK of the
// reduction per wave and step; KS waves sharing an item (KS 4: split
// reduction; 1: a wave per item)
constexpr int kMxMB1 = 1, kMxMB2 = 1;
constexpr int kMxNB1 = 4, kMxNB2 = 4;
constexpr int kMxCK1 = 128, kMxCK2 = 128;
constexpr int kMxKS1 = 4, kMxKS2 = 1;
// From these batch sizes on, items twice as wide (an expert then has enough
// rows that fewer, larger items pay: measured at T = 512 gate/up 86 -> 77 us,
// down 45 -> 41 us; at T <= 128 the narrow gate/up items are faster)
constexpr int kMxWide1T = 256, kMxWide2T = 128;

int nb1_for(int T) { return T >= kMxWide1T ? 2 * kMxNB1 : kMxNB1; }
int nb2_for(int T) { return T >= kMxWide2T ? 2 * kMxNB2 : kMxNB2; }

template <int NB1, int NB2>
hipError_t launch_mx4_nb(const ExpertArgs &a, hipStream_t stream, const Marks *marks, bool gate_up)
{
    const int bm1 = kMxMB1 * 16, bm2 = kMxMB2 * 16;
    const int bn1 = NB1 / 2 * 16, bn2 = NB2 * 16;
    const int cap1 = list_capacity(a.T, a.K, a.E, bm1), cap2 = list_capacity(a.T, a.K, a.E, bm2);
    const int ns1 = a.Is > 0 ? (a.T + bm1 - 1) / bm1 * (a.Is / bn1) : 0;
    const int ns2 = a.Is > 0 ? (a.T + bm2 - 1) / bm2 * (a.H / bn2) : 0;
    const int max1 = ns1 + cap1 * (a.I / bn1);
    const int max2 = ns2 + cap2 * (a.H / bn2);
    const int grid_cap = kMxWgs * max(a.cus, 1);
    // work-groups to cover every item once: an item per work-group (KSPLIT 4) or per wave (1)
    const int g1 = kMxKS1 > 1 ? max1 : (max1 + kWavesMx - 1) / kWavesMx;
    const int g2 = kMxKS2 > 1 ? max2 : (max2 + kWavesMx - 1) / kWavesMx;
    if (gate_up)
        return launch_k(k_expert_stream_mx4<kMxMB1, NB1, kMxCK1, true, kMxKS1>, min(grid_cap, g1), 256,
                        (size_t)(2 * cap1 + a.E + 1 + a.T * a.K) * 4, stream, marks ? marks[0] : Marks{}, a, ns1);
    return launch_k(k_expert_stream_mx4<kMxMB2, NB2, kMxCK2, false, kMxKS2>, min(grid_cap, g2), 256,
                    (size_t)(2 * cap2 + a.E + 1) * 4, stream, marks ? marks[1] : Marks{}, a, ns2);
}
}  // namespace

bool mx4_eligible(int T, int H, int I, int Is)
{
    // every item's reduction splits into its waves x an even number of steps,
    // and every column tile is whole
    const int bn1 = nb1_for(T) / 2 * 16, bn2 = nb2_for(T) * 16;
    return T <= kMx4MaxT && H % (kMxKS1 * 2 * kMxCK1) == 0 && I % (kMxKS2 * 2 * kMxCK2) == 0 &&
           Is % (kMxKS2 * 2 * kMxCK2) == 0 && I % bn1 == 0 && Is % bn1 == 0 && H % bn2 == 0;
}

int mx4_bm1() { return kMxMB1 * 16; }
int mx4_bm2() { return kMxMB2 * 16; }

hipError_t launch_experts_mx4(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    const bool w1 = nb1_for(a.T) != kMxNB1, w2 = nb2_for(a.T) != kMxNB2;
    hipError_t err = w1 ? launch_mx4_nb<2 * kMxNB1, kMxNB2>(a, stream, marks, true)
                        : launch_mx4_nb<kMxNB1, kMxNB2>(a, stream, marks, true);
    if (err != hipSuccess) return err;
    return w2 ? launch_mx4_nb<kMxNB1, 2 * kMxNB2>(a, stream, marks, false)
              : launch_mx4_nb<kMxNB1, kMxNB2>(a, stream, marks, false);
}

}  // namespace flint
