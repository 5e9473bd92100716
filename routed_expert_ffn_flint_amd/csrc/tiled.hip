// LDS-tiled grouped GEMMs for large batches (prefill).
//
// Layer (serving-kit review, "The architecture, from the config"; release news
// page, "What runs on each token"): K selected experts of width I per token plus
// an always-on shared expert of width Is, each a gated three-matrix SwiGLU.
//
// With hundreds of rows per expert the expert products are real GEMMs, so
// operands are staged through LDS and reused:
//   - a work-group computes a 128 x 128 tile (4 waves in 2 x 2, 64 x 64 each,
//     16x16x32 bf16 MFMAs) over k in slices of 64, double-buffered in LDS:
//     the next slice's global loads are in flight while the current slice's
//     MFMAs run;
//   - gate/up tiles hold 64 gate rows and the 64 up rows of the same channels;
//     each wave's columns are 32 gate + the 32 matching up channels, so
//     silu(g) * u is formed in registers;
//   - LDS rows are padded to a 144-byte pitch, which makes the 16-row fragment
//     reads conflict-free;
//   - routed rows are gathered through the expert-sorted token list;
//   - work items are (expert tile, n-tile) with n fastest; a work-group's
//     position is mapped so that consecutive items -- the n-tiles sharing an
//     expert's rows, and the m-tiles sharing its weights -- land on the same
//     XCD (work-groups are spread over the 8 XCDs round-robin), so the shared
//     operand is read from that XCD's L2.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace flint {

namespace {

constexpr int TBM = 128, TBN = 128, TBK = 64;
constexpr int kPitch = TBK + 8;  // bf16 elements per LDS row (144 bytes)
constexpr int kXcds = 8;

// item index seen by this work-group: blockIdx.x % 8 selects the XCD; the
// items of one XCD are consecutive.
__device__ __forceinline__ int xcd_item(int grid)
{
    const int per = grid / kXcds;  // the launcher rounds the grid to a multiple of 8
    return (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
}

}  // namespace

template <bool GATE_UP>
__global__ __launch_bounds__(256, 2) void k_tiled(ExpertArgs a, int n_shared_items)
{
    using S = uint16_t;
    __shared__ __attribute__((aligned(16))) S lds_a[2][TBM * kPitch];
    __shared__ __attribute__((aligned(16))) S lds_b[2][TBN * kPitch];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int H = a.H;

    // ---- the work item
    const int item = xcd_item(gridDim.x);
    const int ntn_shared = GATE_UP ? a.Is / (TBN / 2) : (H + TBN - 1) / TBN;
    const int ntn_routed = GATE_UP ? a.I / (TBN / 2) : (H + TBN - 1) / TBN;
    bool shared = item < n_shared_items;
    int row0, row_end, nt, kdim, e = 0;
    if (shared) {
        row0 = (item / ntn_shared) * TBM;
        nt = item % ntn_shared;
        row_end = a.T;
        kdim = GATE_UP ? H : a.Is;
    } else {
        const int r = item - n_shared_items;
        const int entry = r / ntn_routed;
        const int nlist = GATE_UP ? a.meta[0] : a.meta[1];
        if (entry >= nlist) return;  // (the grid is rounded up past the list's capacity)
        const int32_t *list = GATE_UP ? a.list1 : a.list2;
        e = list[2 * entry];
        row0 = list[2 * entry + 1];
        nt = r % ntn_routed;
        row_end = a.offsets[e + 1];
        kdim = GATE_UP ? H : a.I;
    }

    // ---- global source rows of the 4 A chunks and 4 B chunks this thread copies
    // chunk c = tid + 256*i: row c/8 (0..127), 16-byte column (c%8)
    const int ccol = (tid & 7) * 8;  // element offset within the 64-wide slice
    const S *ga[4];
    const S *gb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = (tid >> 3) + 32 * i;  // tile row
        int r = row0 + rr;
        if (r >= row_end) r = row0;  // padded rows repeat the first row
        if (GATE_UP) {
            const int tok = shared ? r : a.sorted_token[r];
            ga[i] = (const S *)a.x + (size_t)tok * H + ccol;
        } else {
            ga[i] = (shared ? (const S *)a.h_shared : (const S *)a.h_sorted) + (size_t)r * kdim + ccol;
        }
        if (GATE_UP) {
            // B rows 0..63: gate channels nt*64 + rr; rows 64..127: the same up channels
            const int ch = nt * 64 + (rr & 63);
            const S *w = shared ? (rr < 64 ? (const S *)a.shared_gate : (const S *)a.shared_up)
                                : (rr < 64 ? (const S *)a.gate : (const S *)a.up) + (size_t)e * a.I * H;
            gb[i] = w + (size_t)ch * H + ccol;
        } else {
            int c = nt * TBN + rr;
            if (c >= H) c = 0;
            const S *w = shared ? (const S *)a.shared_down : (const S *)a.down + (size_t)e * H * a.I;
            gb[i] = w + (size_t)c * kdim + ccol;
        }
    }

    u32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *reinterpret_cast<const u32x4 *>(ga[i] + k0);
            rb[i] = *reinterpret_cast<const u32x4 *>(gb[i] + k0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = (tid >> 3) + 32 * i;
            *reinterpret_cast<u32x4 *>(&lds_a[buf][rr * kPitch + ccol]) = ra[i];
            *reinterpret_cast<u32x4 *>(&lds_b[buf][rr * kPitch + ccol]) = rb[i];
        }
    };

    // ---- wave fragments: 4 row blocks (A) x 4 column blocks (B) of 16
    // A rows: wm*64 + m*16 + (lane&15).  B rows (GATE_UP): gate blocks j<2 at
    // wn*32 + j*16, up blocks j>=2 at 64 + wn*32 + (j-2)*16; (down) wn*64 + j*16.
    int boff[4], aoff[4];
    const int kq = (lane >> 4) * 8;
#pragma unroll
    for (int m = 0; m < 4; ++m) aoff[m] = (wm * 64 + m * 16 + (lane & 15)) * kPitch + kq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int br = GATE_UP ? (j < 2 ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16) : wn * 64 + j * 16;
        boff[j] = (br + (lane & 15)) * kPitch + kq;
    }

    f32x4 acc[4][4];
    zero_acc(acc);
    const int nk = kdim / TBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * TBK);
#pragma unroll
        for (int kk = 0; kk < TBK; kk += 32) {
            Frag<BF16> fa[4], fb[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) fa[m].load(&lds_a[buf][aoff[m] + kk]);
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j].load(&lds_b[buf][boff[j] + kk]);
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) mma(acc[m][j], fa[m], fb[j]);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = row0 + wm * 64 + m * 16 + (lane >> 4) * 4 + i;
            if (r >= row_end || r >= row0 + TBM) continue;
            if (GATE_UP) {
                S *hout = shared ? (S *)a.h_shared : (S *)a.h_sorted;
                const int width = shared ? a.Is : a.I;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int ch = nt * 64 + wn * 32 + j * 16 + (lane & 15);
                    hout[(size_t)r * width + ch] = f32_to_bf16(swiglu(acc[m][j][i], acc[m][j + 2][i]));
                }
            } else {
                float *yout = shared ? a.y_shared : a.y_sorted;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = nt * TBN + wn * 64 + j * 16 + (lane & 15);
                    if (c < H) yout[(size_t)r * H + c] = acc[m][j][i];
                }
            }
        }
    }
}

bool tiled_eligible(int H, int I, int Is, bool bf16)
{
    // k slices of 64; gate/up tiles of 64 channels
    return bf16 && H % TBK == 0 && I % 64 == 0 && Is % 64 == 0;
}

hipError_t launch_experts_tiled(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    const int cap1 = list_capacity(a.T, a.K, a.E, TBM);
    const int cap2 = cap1;
    const int mt = (a.T + TBM - 1) / TBM;
    const int ns1 = a.Is > 0 ? mt * (a.Is / (TBN / 2)) : 0;
    const int ns2 = a.Is > 0 ? mt * ((a.H + TBN - 1) / TBN) : 0;
    auto round8 = [](int g) { return (g + kXcds - 1) / kXcds * kXcds; };
    const int g1 = round8(ns1 + cap1 * (a.I / (TBN / 2)));
    const int g2 = round8(ns2 + cap2 * ((a.H + TBN - 1) / TBN));
    const hipError_t err = launch_k(k_tiled<true>, g1, 256, 0, stream, marks ? marks[0] : Marks{}, a, ns1);
    if (err != hipSuccess) return err;
    return launch_k(k_tiled<false>, g2, 256, 0, stream, marks ? marks[1] : Marks{}, a, ns2);
}

}  // namespace flint
