// Expert kernels of the Flint MoE layer (gfx950): grouped gate/up GEMM with a
// fused SwiGLU, grouped down GEMM, weighted combine.
//
// Layer (serving-kit review, "The architecture, from the config"; release news
// page, "What runs on each token"): each token runs its K selected experts of
// width I and an always-on shared expert of width Is; the gated three-matrix
// expert form fits the serving-kit review's parameter count.
//
//   k_gate_up  h[slot][c] = silu(gate[e][c] . x[tok]) * (up[e][c] . x[tok])  -> dtype
//              routed rows are gathered through sorted_token; the shared expert
//              is the same kernel over all T tokens with its own weights.
//   k_down     y[slot][n] = down[e][n] . h[slot]                             -> float32
//   k_combine  out[t] = sum_k w[t][k] * y[slot_of[t][k]] + y_shared[t]        -> out dtype
//
// Work items: the shared expert's tiles come first (their number is known on
// the host), then the routed tiles listed on the device by the dispatch
// kernel.  The grid covers the list's capacity; items past the list's actual
// length exit at once, so the host never reads a device count.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace flint {

// Small-batch tile shapes (decode): rows per tile 32 (MB = 2 blocks of 16),
// split-k over SPLIT waves.  Gate/up: NB/2 channels-blocks of 16 per tile;
// down: NB column blocks of 16 per tile.
constexpr int kGuNb = 4;
constexpr int kGuSplit = 4;
constexpr int kGuUnroll = 4;
constexpr int kDnNb = 4;
constexpr int kDnSplit = 4;
constexpr int kDnUnroll = 4;
constexpr bool kGuPipe = false;
constexpr bool kDnPipe = false;

template <int SPLIT> struct WaveGrid {  // SPLIT waves, same tile, k split SPLIT ways
    static constexpr int WM = 1, WN = 1, THREADS = SPLIT * 64;
};
template <> struct WaveGrid<1> {  // 4 waves in a 2x2 grid, all of k each
    static constexpr int WM = 2, WN = 2, THREADS = 256;
};

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU.  A wave's NB column blocks are NB/2 gate blocks and the NB/2
// up blocks of the same channels, so silu(g)*u pairs up in registers.
template <typename DT, int MB, int NB, int SPLIT, int U, bool PIPE>
__global__ __launch_bounds__(WaveGrid<SPLIT>::THREADS) void k_gate_up(ExpertArgs a, int n_shared_items)
{
    using S = typename DT::storage;
    constexpr bool SPLITK = SPLIT > 1;
    constexpr int WM = WaveGrid<SPLIT>::WM, WN = WaveGrid<SPLIT>::WN;
    constexpr int BM = WM * MB * 16, HALF = NB / 2, BN = WN * HALF * 16;
    __shared__ float red[SPLITK ? SPLIT * MB * NB * 256 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = SPLITK ? 0 : wave / WN, wn = SPLITK ? 0 : wave % WN;
    const int H = a.H;
    const S *x = (const S *)a.x;

    int item = blockIdx.x;
    const bool shared = item < n_shared_items;
    int width, row0, n0, e = -1, row_end = a.T;
    const S *wg, *wu;
    S *hout;
    if (shared) {
        const int ntn = a.Is / BN;
        row0 = (item / ntn) * BM;
        n0 = (item % ntn) * BN;
        width = a.Is;
        wg = (const S *)a.shared_gate;
        wu = (const S *)a.shared_up;
        hout = (S *)a.h_shared;
    } else {
        item -= n_shared_items;
        const int ntn = a.I / BN;
        const int entry = item / ntn;
        const int nlist = a.K == 0 ? 0 : a.meta[0];
        e = a.list1[2 * entry];  // inside the list's capacity; used only if entry < nlist
        row0 = a.list1[2 * entry + 1];
        if (entry >= nlist) return;
        row_end = a.offsets[e + 1];
        n0 = (item % ntn) * BN;
        width = a.I;
        wg = (const S *)a.gate + (size_t)e * a.I * H;
        wu = (const S *)a.up + (size_t)e * a.I * H;
        hout = (S *)a.h_sorted;
    }

    const int kg = (lane >> 4) * 8;
    const int rbase = row0 + wm * MB * 16;
    const int cbase = n0 + wn * HALF * 16;
    const S *b_rows[NB];
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
        const int c = cbase + j * 16 + (lane & 15);
        b_rows[j] = wg + (size_t)c * H + kg;
        b_rows[j + HALF] = wu + (size_t)c * H + kg;
    }
    // A rows: routed rows are gathered token rows; rows past the tile's end
    // repeat its first row (cache hits; their results are never stored)
    auto resolve_a = [&](const S *(&a_rows)[MB]) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            int r = rbase + m * 16 + (lane & 15);
            if (r >= row_end) r = row0;
            const int tok = shared ? r : a.sorted_token[r];
            a_rows[m] = x + (size_t)tok * H + kg;
        }
    };

    f32x4 acc[MB][NB];
    zero_acc(acc);
    const int nslices = H / 32;
    int s0 = 0, s1 = nslices;
    if (SPLITK) {
        const int per = (nslices + SPLIT - 1) / SPLIT;
        s0 = min(wave * per, nslices);
        s1 = min(s0 + per, nslices);
    }
    wave_gemm_stream<DT, MB, NB, U, PIPE>(resolve_a, b_rows, s0, s1, acc);
    if (SPLITK) splitk_reduce<SPLIT, MB, NB>(acc, red);

#pragma unroll
    for (int j = 0; j < HALF; ++j) {
        if (SPLITK && (j % SPLIT) != wave) continue;  // spread the stores over the waves
        const int c = cbase + j * 16 + (lane & 15);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rbase + m * 16 + (lane >> 4) * 4 + i;
                if (r < row_end)
                    store_elem<DT>(hout + (size_t)r * width + c, swiglu(acc[m][j][i], acc[m][j + HALF][i]));
            }
    }
}

// ---------------------------------------------------------------------------
// Down projection: y[row][n] = down[n] . h[row], float32 out.
template <typename DT, int MB, int NB, int SPLIT, int U, bool PIPE>
__global__ __launch_bounds__(WaveGrid<SPLIT>::THREADS) void k_down(ExpertArgs a, int n_shared_items)
{
    using S = typename DT::storage;
    constexpr bool SPLITK = SPLIT > 1;
    constexpr int WM = WaveGrid<SPLIT>::WM, WN = WaveGrid<SPLIT>::WN;
    constexpr int BM = WM * MB * 16, BN = WN * NB * 16;
    __shared__ float red[SPLITK ? SPLIT * MB * NB * 256 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = SPLITK ? 0 : wave / WN, wn = SPLITK ? 0 : wave % WN;
    const int H = a.H;
    const int ntn = (H + BN - 1) / BN;

    int item = blockIdx.x;
    const bool shared = item < n_shared_items;
    int kdim, row0, n0, e = -1, row_end = a.T;
    const S *hin, *wd;
    float *yout;
    if (shared) {
        row0 = (item / ntn) * BM;
        n0 = (item % ntn) * BN;
        kdim = a.Is;
        hin = (const S *)a.h_shared;
        wd = (const S *)a.shared_down;
        yout = a.y_shared;
    } else {
        item -= n_shared_items;
        const int entry = item / ntn;
        const int nlist = a.K == 0 ? 0 : a.meta[1];
        e = a.list2[2 * entry];
        row0 = a.list2[2 * entry + 1];
        if (entry >= nlist) return;
        row_end = a.offsets[e + 1];
        n0 = (item % ntn) * BN;
        kdim = a.I;
        hin = (const S *)a.h_sorted;
        wd = (const S *)a.down + (size_t)e * H * a.I;
        yout = a.y_sorted;
    }

    const int kg = (lane >> 4) * 8;
    const int rbase = row0 + wm * MB * 16;
    const int cbase = n0 + wn * NB * 16;
    const S *b_rows[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        int c = cbase + n * 16 + (lane & 15);
        if (c >= H) c = 0;
        b_rows[n] = wd + (size_t)c * kdim + kg;
    }
    auto resolve_a = [&](const S *(&a_rows)[MB]) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            int r = rbase + m * 16 + (lane & 15);
            if (r >= row_end) r = row0;
            a_rows[m] = hin + (size_t)r * kdim + kg;
        }
    };

    f32x4 acc[MB][NB];
    zero_acc(acc);
    const int nslices = kdim / 32;
    int s0 = 0, s1 = nslices;
    if (SPLITK) {
        const int per = (nslices + SPLIT - 1) / SPLIT;
        s0 = min(wave * per, nslices);
        s1 = min(s0 + per, nslices);
    }
    wave_gemm_stream<DT, MB, NB, U, PIPE>(resolve_a, b_rows, s0, s1, acc);
    if (SPLITK) splitk_reduce<SPLIT, MB, NB>(acc, red);

#pragma unroll
    for (int n = 0; n < NB; ++n) {
        if (SPLITK && (n % SPLIT) != wave) continue;
        const int c = cbase + n * 16 + (lane & 15);
        if (c >= H) continue;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rbase + m * 16 + (lane >> 4) * 4 + i;
                if (r < row_end) yout[(size_t)r * H + c] = acc[m][n][i];
            }
    }
}

// ---------------------------------------------------------------------------
// out[t] = sum_k w[t][k] * y_sorted[slot_of[t*K+k]] + y_shared[t]   (fixed order)
// Y16: y_sorted and a single y_shared hold fp16 values times 2^y_scale (see
// ExpertArgs::y16).
// combine4: columns c .. c+3 of token t (c a multiple of 4, below H).
template <bool Y16>
__device__ __forceinline__ f32x4 combine4(const ExpertArgs &a, int t, int c)
{
    const int H = a.H, K = a.K;
    // Every load is issued before any is used (entries past K re-read entry
    // K-1, rows past them are not added): the rows arrive in one memory
    // latency instead of one each.
    int slots[kMaxTopK];
    float w[kMaxTopK];
    f32x4 y[kMaxTopK];
    if (K > 0) {  // K = 0: a dense layer, the shared term alone
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            const size_t i = (size_t)t * K + (k < K ? k : K - 1);
            slots[k] = a.slot_of[i];
            w[k] = a.topk_w[i];
        }
        if (Y16) {
            typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
            const _Float16 *y16 = reinterpret_cast<const _Float16 *>(a.y_sorted);
            h16x4 v[kMaxTopK];
            int8_t sc[kMaxTopK];
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                v[k] = *reinterpret_cast<const h16x4 *>(y16 + (size_t)slots[k] * H + c);
                sc[k] = a.y_scale[(size_t)slots[k] * (H / kYScaleCols) + c / kYScaleCols];
            }
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k)
#pragma unroll
                for (int j = 0; j < 4; ++j) y[k][j] = ldexpf((float)v[k][j], sc[k]);
        } else {
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k)
                y[k] = *reinterpret_cast<const f32x4 *>(a.y_sorted + (size_t)slots[k] * H + c);
        }
    }
    const int nsplit = a.shared_splits > 1 ? a.shared_splits : 1;
    f32x4 ys = {0.f, 0.f, 0.f, 0.f};
    if (Y16 && a.Is > 0 && nsplit == 1) {  // fp16 times 2^exponent, the exponents after the T*K routed rows
        typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
        const h16x4 v = *reinterpret_cast<const h16x4 *>(reinterpret_cast<const _Float16 *>(a.y_shared) +
                                                         (size_t)t * H + c);
        const int sc = a.y_scale[((size_t)a.T * K + t) * (H / kYScaleCols) + c / kYScaleCols];
#pragma unroll
        for (int j = 0; j < 4; ++j) ys[j] = ldexpf((float)v[j], sc);
    } else if (a.Is > 0) {
        ys = *reinterpret_cast<const f32x4 *>(a.y_shared + (size_t)t * H + c);
    }
    // the shared down product's other partial sums, loaded together here and
    // added in order below (one memory latency for all of them instead of one
    // each: a dense T = 32 layer's combine of 8 partial arrays 4.6 -> 3.4 us)
    constexpr int kPre = 8;
    f32x4 ps[kPre - 1];
    if (a.Is > 0 && nsplit > 1) {
#pragma unroll
        for (int sp = 1; sp < kPre; ++sp)
            if (sp < nsplit) ps[sp - 1] = *reinterpret_cast<const f32x4 *>(a.y_shared + ((size_t)sp * a.T + t) * H + c);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        if (k < K) {
            acc[0] += w[k] * y[k][0];
            acc[1] += w[k] * y[k][1];
            acc[2] += w[k] * y[k][2];
            acc[3] += w[k] * y[k][3];
        }
    }
    if (a.Is > 0) {
        acc[0] += ys[0];
        acc[1] += ys[1];
        acc[2] += ys[2];
        acc[3] += ys[3];
#pragma unroll
        for (int sp = 1; sp < kPre; ++sp) {
            if (sp >= nsplit) break;
            acc[0] += ps[sp - 1][0];
            acc[1] += ps[sp - 1][1];
            acc[2] += ps[sp - 1][2];
            acc[3] += ps[sp - 1][3];
        }
        for (int sp = kPre; sp < nsplit; ++sp) {  // (more than kPre partial arrays: the rest one by one)
            const f32x4 v = *reinterpret_cast<const f32x4 *>(a.y_shared + ((size_t)sp * a.T + t) * H + c);
            acc[0] += v[0];
            acc[1] += v[1];
            acc[2] += v[2];
            acc[3] += v[3];
        }
    }
    if (a.fail && *a.fail) {  // a wait of the fused decode kernel gave up: the result is void
        const float nan = __builtin_nanf("");
        acc = f32x4{nan, nan, nan, nan};
    }
    return acc;
}

__device__ __forceinline__ void store_out4(const ExpertArgs &a, int t, int c, f32x4 acc)
{
    if (a.out_bf16) {
        uint16_t *o = (uint16_t *)a.out + (size_t)t * a.H + c;
        o[0] = f32_to_bf16(acc[0]);
        o[1] = f32_to_bf16(acc[1]);
        o[2] = f32_to_bf16(acc[2]);
        o[3] = f32_to_bf16(acc[3]);
    } else {
        *reinterpret_cast<f32x4 *>((float *)a.out + (size_t)t * a.H + c) = acc;
    }
}

template <bool Y16>
__global__ __launch_bounds__(256) void k_combine(ExpertArgs a)
{
    const int t = blockIdx.x;
    const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
    if (c >= a.H) return;
    store_out4(a, t, c, combine4<Y16>(a, t, c));
}

// ---------------------------------------------------------------------------
ExpertTiles expert_tiles_for(int T, int H, int E, int K, int I, int Is, bool bf16)
{
    // the LDS-tiled kernels: a bf16 dense layer at every T, a MoE layer from
    // kTiledFromT rows (their tile rows depend on T: tiled_bm1 / tiled_bm2)
    if (tiled_eligible(T, K, E, H, I, Is, bf16) && (K == 0 || T >= kTiledFromT))
        return ExpertTiles{tiled_bm1(T, K, E, Is), 0, tiled_bm2(T, K, E), 0, false, false, true};
    if (T <= kStreamMaxT) {
        if (stream_eligible(T, H, I, Is))
            return ExpertTiles{stream_bm1(T, K), 0, stream_bm2(), 0, true, true, false};
        // Small batches (decode): split-k kernels over 32-row tiles, so that one
        // tile holds every row an expert gets and each weight is read once.
        return ExpertTiles{32, kGuNb / 2 * 16, 32, kDnNb * 16, true, false, false};
    }
    return ExpertTiles{128, 64, 128, 128, false, false, false};
}

template <typename DT>
static hipError_t launch_experts_t(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    const ExpertTiles &t = a.tiles;
    const Marks m1 = marks ? marks[0] : Marks{}, m2 = marks ? marks[1] : Marks{}, m3 = marks ? marks[2] : Marks{};
    if (a.mx4) {
        const hipError_t err = launch_experts_mx4(a, stream, marks);
        if (err != hipSuccess) return err;
        return a.skip_combine ? hipSuccess : launch_combine(a, stream, m3);
    }
    if (t.stream || t.tiled) {
        // the tiled down product stores the routed rows as scaled fp16
        ExpertArgs b = a;
        b.y16 = t.tiled && a.K > 0;
        const hipError_t err =
            t.stream ? launch_experts_stream(b, stream, marks) : launch_experts_tiled(b, stream, marks);
        if (err != hipSuccess) return err;
        return b.skip_combine ? hipSuccess : launch_combine(b, stream, m3);
    }
    const int cap1 = list_capacity(a.T, a.K, a.E, t.bm1);
    const int cap2 = list_capacity(a.T, a.K, a.E, t.bm2);
    const int mt1 = (a.T + t.bm1 - 1) / t.bm1, mt2 = (a.T + t.bm2 - 1) / t.bm2;
    const int ns1 = a.Is > 0 ? mt1 * (a.Is / t.bn1) : 0;
    const int ns2 = a.Is > 0 ? mt2 * ((a.H + t.bn2 - 1) / t.bn2) : 0;
    const int g1 = ns1 + cap1 * (a.I / t.bn1);
    const int g2 = ns2 + cap2 * ((a.H + t.bn2 - 1) / t.bn2);
    hipError_t err;
    if (t.small)
        err = launch_k(k_gate_up<DT, 2, kGuNb, kGuSplit, kGuUnroll, kGuPipe>, g1,
                       WaveGrid<kGuSplit>::THREADS, 0, stream, m1, a, ns1);
    else
        err = launch_k(k_gate_up<DT, 4, 4, 1, 4, false>, g1, 256, 0, stream, m1, a, ns1);
    if (err != hipSuccess) return err;
    if (t.small)
        err = launch_k(k_down<DT, 2, kDnNb, kDnSplit, kDnUnroll, kDnPipe>, g2,
                       WaveGrid<kDnSplit>::THREADS, 0, stream, m2, a, ns2);
    else
        err = launch_k(k_down<DT, 4, 4, 1, 4, false>, g2, 256, 0, stream, m2, a, ns2);
    if (err != hipSuccess) return err;
    return a.skip_combine ? hipSuccess : launch_combine(a, stream, m3);
}


hipError_t launch_experts(const ExpertArgs &a, hipStream_t stream, const Marks *marks)
{
    if (a.T <= 0) return hipSuccess;
    return a.bf16 ? launch_experts_t<BF16>(a, stream, marks) : launch_experts_t<F32>(a, stream, marks);
}

// ---------------------------------------------------------------------------
// RMSNorm between stacked layers: out = bf16(in / sqrt(mean(in^2) + eps)).
// Sum of squares and the scaling in double; the double result is rounded to
// float with round-to-odd and then to bf16 with round-to-nearest-even, which
// together round the double once to nearest-even bf16.
__device__ __forceinline__ uint16_t f64_to_bf16(double d)
{
    float f = (float)d;
    if ((double)f != d) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(d)) u -= 1u;  // step back toward zero
        u |= 1u;
        f = __uint_as_float(u);
    }
    return f32_to_bf16(f);
}

// One row by a work-group of 256 threads (row in global memory or LDS): the
// sum of squares in the same order wherever the row lies, so the result has
// the same bits.  part: 4 doubles of LDS.
__device__ __forceinline__ void rmsnorm_row(const float *row, int H, float eps, uint16_t *__restrict__ out,
                                            double *part)
{
    double ss = 0.0;
    for (int c = threadIdx.x; c < H; c += 256) ss += (double)row[c] * (double)row[c];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = part[0] + part[1] + part[2] + part[3];
    const double r = 1.0 / sqrt(tot / (double)H + (double)eps);
    for (int c = threadIdx.x; c < H; c += 256) out[c] = f64_to_bf16((double)row[c] * r);
}

__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ in, int H, float eps,
                                                 uint16_t *__restrict__ out)
{
    __shared__ double part[4];
    const int t = blockIdx.x;
    rmsnorm_row(in + (size_t)t * H, H, eps, out + (size_t)t * H, part);
}

// The combine of one token row, then RMSNorm of its float32 sums into
// a.norm_out, in one work-group: the row goes through LDS (H floats of
// dynamic LDS), where the norm reads it in k_rmsnorm's order, so the bits are
// those of k_rmsnorm on the float32 output.
template <bool Y16>
__global__ __launch_bounds__(256) void k_combine_rmsnorm(ExpertArgs a)
{
    extern __shared__ float row[];
    __shared__ double part[4];
    const int t = blockIdx.x;
    for (int c = threadIdx.x * 4; c < a.H; c += 256 * 4) {
        const f32x4 acc = combine4<Y16>(a, t, c);
        store_out4(a, t, c, acc);
        *reinterpret_cast<f32x4 *>(row + c) = acc;
    }
    __syncthreads();
    rmsnorm_row(row, a.H, a.norm_eps, a.norm_out + (size_t)t * a.H, part);
}

hipError_t launch_combine(const ExpertArgs &a, hipStream_t stream, Marks m)
{
    if (a.T <= 0) return hipSuccess;
    if (a.norm_out) {
        const size_t lds = (size_t)a.H * 4;
        return a.y16 ? launch_k(k_combine_rmsnorm<true>, a.T, 256, lds, stream, m, a)
                     : launch_k(k_combine_rmsnorm<false>, a.T, 256, lds, stream, m, a);
    }
    const dim3 grid(a.T, (a.H + 1023) / 1024);
    return a.y16 ? launch_k(k_combine<true>, grid, 256, 0, stream, m, a)
                 : launch_k(k_combine<false>, grid, 256, 0, stream, m, a);
}

hipError_t launch_rmsnorm(int T, int H, const float *in, uint16_t *out, float eps, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    k_rmsnorm<<<T, 256, 0, stream>>>(in, H, eps, out);
    return hipGetLastError();
}

}  // namespace flint
