// Persistent weight-streaming expert kernels for block-scaled 4-bit expert
// weights (MXFP4), small batches.
//
// Layer (serving-kit review, "The architecture, from the config"; release news
// page, "What runs on each token"): K selected experts of width I per token plus
// an always-on shared expert of width Is, each a gated three-matrix SwiGLU.
// Weight format (a definition; the pages' low-bit builds store 4-bit weights,
// release news, "Availability"): OCP Microscaling MXFP4 -- FP4 E2M1 elements,
// 32-element blocks along the reduction dimension, an E8M0 scale 2^(s-127) per
// block, two elements per byte with the lower-indexed one in the low nibble.
//
// Same structure as the bf16 streaming kernels (persistent grid, tile list in
// LDS, four waves splitting the reduction dimension, ping-pong buffers, partial
// sums added in wave order), with the weight side 4-bit:
//   - a step covers CK values of k per wave; lane group g (lane >> 4) takes
//     elements [k0 + g*CK/4, +CK/4) of its row, which lie in one 32-element
//     block: CK/8 bytes of codes and one scale byte per weight row, loaded as
//     one vector and one byte;
//   - the activations use the same assignment of k to lanes, so MFMA j of the
//     step multiplies elements k0 + g*CK/4 + 8j .. +7 on both sides (the k
//     order of the sum is permuted, its value is not);
//   - v_cvt_scalef32_pk_bf16_fp4 turns two codes into two bf16 values times
//     the block scale, exactly (E2M1 x 2^n is a bf16 value), so the MFMAs are
//     the bf16 ones and everything after them is as in the bf16 path.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace flint {

namespace {

constexpr int kWavesMx = 4;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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
template <int CK> struct CodeVec;
template <> struct CodeVec<64> {
    uint32_t w[2];
    __device__ __forceinline__ void load(const uint8_t *p)
    {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        w[0] = v.x;
        w[1] = v.y;
    }
};
template <> struct CodeVec<128> {
    uint32_t w[4];
    __device__ __forceinline__ void load(const uint8_t *p)
    {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
        w[0] = v[0];
        w[1] = v[1];
        w[2] = v[2];
        w[3] = v[3];
    }
};

// What one wave needs for one work item.
template <int MB, int NB>
struct MxItem {
    const uint16_t *a[MB];  // activation rows, at this lane's k offset
    const uint8_t *q[NB];   // weight code rows, at this lane's k offset
    const uint8_t *s[NB];   // weight scale rows, at this lane's block
    int nstep;              // steps of this wave
    int row0, row_end, n0, shared, valid;
};

}  // namespace

// GATE_UP: gate/up + SwiGLU -> h (bf16);  otherwise: down -> y (float32).
// MB row blocks of 16, NB column blocks of 16 (gate/up: NB/2 gate + NB/2 up).
template <int MB, int NB, int CK, bool GATE_UP>
__global__ __launch_bounds__(256, 2) void k_expert_stream_mx4(ExpertArgs a, int n_shared_items)
{
    constexpr int BM = MB * 16;
    constexpr int HALF = NB / 2;
    constexpr int BN = GATE_UP ? HALF * 16 : NB * 16;
    constexpr int NF = CK / 32;  // fragments (MFMA k-steps) per step
    extern __shared__ int32_t dyn_lds[];
    __shared__ float red[kWavesMx * MB * NB * 256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int H = a.H;
    const int nlist = GATE_UP ? a.meta[0] : a.meta[1];
    int32_t *list = dyn_lds;
    int32_t *offsets = dyn_lds + 2 * nlist;
    for (int i = threadIdx.x; i < 2 * nlist; i += blockDim.x) list[i] = (GATE_UP ? a.list1 : a.list2)[i];
    for (int i = threadIdx.x; i <= a.E; i += blockDim.x) offsets[i] = a.offsets[i];
    __syncthreads();

    const int ntn_shared = GATE_UP ? a.Is / BN : (H + BN - 1) / BN;
    const int ntn_routed = GATE_UP ? a.I / BN : (H + BN - 1) / BN;
    const int n_items = n_shared_items + nlist * ntn_routed;

    auto get = [&](int item) {
        MxItem<MB, NB> it;
        it.valid = item < n_items;
        if (!it.valid) item = 0;  // a valid item's addresses, used only as dummy prefetch targets
        int e = 0, nt, kdim;
        const uint8_t *qa, *qb, *sa, *sb;  // codes / scales: gate, up (GATE_UP) or down (qa, sa)
        if (item < n_shared_items) {
            it.shared = 1;
            it.row0 = (item / ntn_shared) * BM;
            nt = item % ntn_shared;
            it.row_end = a.T;
            kdim = GATE_UP ? H : a.Is;
            qa = (const uint8_t *)(GATE_UP ? a.shared_gate : a.shared_down);
            sa = GATE_UP ? a.shared_gate_s : a.shared_down_s;
            qb = (const uint8_t *)a.shared_up;
            sb = a.shared_up_s;
        } else {
            it.shared = 0;
            const int r = item - n_shared_items;
            const int entry = r / ntn_routed;
            nt = r % ntn_routed;
            e = list[2 * entry];
            it.row0 = list[2 * entry + 1];
            it.row_end = offsets[e + 1];
            kdim = GATE_UP ? H : a.I;
            const size_t rows_before = (size_t)e * (GATE_UP ? a.I : H);  // weight rows of earlier experts
            qa = (const uint8_t *)(GATE_UP ? a.gate : a.down) + rows_before * (kdim / 2);
            sa = (GATE_UP ? a.gate_s : a.down_s) + rows_before * (kdim / 32);
            qb = (const uint8_t *)a.up + rows_before * (kdim / 2);
            sb = a.up_s + rows_before * (kdim / 32);
        }
        it.n0 = nt * BN;
        it.nstep = kdim / CK / kWavesMx;  // the launcher checks divisibility (and evenness)
        const int kw = wave * it.nstep * CK + g * (CK / 4);  // this lane's first k
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            int c = GATE_UP ? it.n0 + (n % HALF) * 16 + (lane & 15) : it.n0 + n * 16 + (lane & 15);
            if (!GATE_UP && c >= H) c = 0;
            const bool up = GATE_UP && n >= HALF;
            it.q[n] = (up ? qb : qa) + (size_t)c * (kdim / 2) + kw / 2;
            it.s[n] = (up ? sb : sa) + (size_t)c * (kdim / 32) + kw / 32;
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            int r = it.row0 + m * 16 + (lane & 15);
            if (r >= it.row_end) r = it.row0;  // rows past the tile repeat its first row (cache hits)
            if (GATE_UP) {
                const int tok = it.shared ? r : a.sorted_token[r];
                it.a[m] = (const uint16_t *)a.x + (size_t)tok * H + kw;
            } else {
                it.a[m] = (it.shared ? (const uint16_t *)a.h_shared : (const uint16_t *)a.h_sorted) +
                          (size_t)r * kdim + kw;
            }
        }
        return it;
    };

    // raw step buffers: activation fragments, weight codes, scale bytes
    struct Raw {
        Frag<BF16> fa[MB][NF];
        CodeVec<CK> q[NB];
        uint32_t s[NB];
    };
    auto load = [&](const MxItem<MB, NB> &it, int step, Raw &r) {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            r.q[n].load(it.q[n] + step * (CK / 2));
            r.s[n] = it.s[n][step * (CK / 32)];
        }
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < NF; ++j) r.fa[m][j].load(it.a[m] + step * CK + 8 * j);
    };
    f32x4 acc[MB][NB];
    auto compute = [&](const Raw &r) {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const float sc = e8m0_to_f32(r.s[n]);
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                Frag<BF16> fb;
                fp4x8_to_frag(r.q[n].w[j], sc, fb);
#pragma unroll
                for (int m = 0; m < MB; ++m) mma(acc[m][n], r.fa[m][j], fb);
            }
        }
    };

    int item = blockIdx.x;
    MxItem<MB, NB> cur = get(item);
    if (!cur.valid) return;  // uniform across the work-group
    Raw ra, rb;
    load(cur, 0, ra);
    while (true) {
        const MxItem<MB, NB> nxt = get(item + gridDim.x);
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
        splitk_reduce<kWavesMx, MB, NB>(acc, red);
        if (GATE_UP) {
            uint16_t *hout = cur.shared ? (uint16_t *)a.h_shared : (uint16_t *)a.h_sorted;
            const int width = cur.shared ? a.Is : a.I;
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                if ((j % kWavesMx) != wave) continue;
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
                if ((n % kWavesMx) != wave) continue;
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

namespace {
constexpr int kMxMB = 2, kMxNB1 = 4, kMxNB2 = 2, kMxCK1 = 128, kMxCK2 = 64;
}

bool mx4_eligible(int T, int H, int I, int Is)
{
    // every item's reduction splits into 4 waves x an even number of steps
    return T <= kMx4MaxT && H % (kWavesMx * 2 * kMxCK1) == 0 && I % (kWavesMx * 2 * kMxCK2) == 0 &&
           Is % (kWavesMx * 2 * kMxCK2) == 0 && I % (kMxNB1 / 2 * 16) == 0 && Is % (kMxNB1 / 2 * 16) == 0;
}

int mx4_bm() { return kMxMB * 16; }

hipError_t launch_experts_mx4(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    const int bm = kMxMB * 16;
    const int bn1 = kMxNB1 / 2 * 16, bn2 = kMxNB2 * 16;
    const int cap = list_capacity(a.T, a.K, a.E, bm);
    const int mt = (a.T + bm - 1) / bm;
    const int ns1 = a.Is > 0 ? mt * (a.Is / bn1) : 0;
    const int ns2 = a.Is > 0 ? mt * ((a.H + bn2 - 1) / bn2) : 0;
    const int max1 = ns1 + cap * (a.I / bn1);
    const int max2 = ns2 + cap * ((a.H + bn2 - 1) / bn2);
    const size_t lds = (size_t)(2 * cap + a.E + 1) * 4;
    const int grid_cap = 2 * max(a.cus, 1);
    hipError_t err = launch_k(k_expert_stream_mx4<kMxMB, kMxNB1, kMxCK1, true>, min(grid_cap, max1), 256, lds, stream,
                              marks ? marks[0] : Marks{}, a, ns1);
    if (err != hipSuccess) return err;
    return launch_k(k_expert_stream_mx4<kMxMB, kMxNB2, kMxCK2, false>, min(grid_cap, max2), 256, lds, stream,
                    marks ? marks[1] : Marks{}, a, ns2);
}

}  // namespace flint
