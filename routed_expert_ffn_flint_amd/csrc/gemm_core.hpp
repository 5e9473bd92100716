// Wave-level MFMA tile loop shared by the router, gate/up and down kernels.
//
// A wave accumulates an (MB*16) x (NB*16) fp32 tile over a range of 32-wide
// k slices.  Operands are streamed from global memory straight into registers:
// each lane loads, per slice, 8 consecutive elements of its A row and of its B
// row (16 B for bf16).  A rows are activations (tokens), B rows are weight rows
// ([out][in] layout, so both operands are contiguous along k).  There is no
// LDS staging: every weight element is used by exactly one MFMA column, and
// for the small-M shapes of decode there is nothing to share.
#pragma once

#include "common.hpp"

namespace flint {

// a_rows[m]: lane's A row pointer for m-block m (row = m*16 + (lane & 15)),
//            already offset by the lane's k group (8 * (lane >> 4)).
// b_rows[n]: same for B (column n*16 + (lane & 15)).
// Slices [s0, s1) of 32 elements each.
template <typename DT, int MB, int NB, int UNROLL>
__device__ __forceinline__ void wave_gemm(const typename DT::storage *const (&a_rows)[MB],
                                          const typename DT::storage *const (&b_rows)[NB],
                                          int s0, int s1, f32x4 (&acc)[MB][NB])
{
    int s = s0;
    for (; s + UNROLL <= s1; s += UNROLL) {
        Frag<DT> a[UNROLL][MB];
        Frag<DT> b[UNROLL][NB];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
            for (int n = 0; n < NB; ++n) b[u][n].load(b_rows[n] + (s + u) * 32);
#pragma unroll
            for (int m = 0; m < MB; ++m) a[u][m].load(a_rows[m] + (s + u) * 32);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int n = 0; n < NB; ++n) mma(acc[m][n], a[u][m], b[u][n]);
    }
    for (; s < s1; ++s) {
        Frag<DT> a[MB];
        Frag<DT> b[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) b[n].load(b_rows[n] + s * 32);
#pragma unroll
        for (int m = 0; m < MB; ++m) a[m].load(a_rows[m] + s * 32);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int n = 0; n < NB; ++n) mma(acc[m][n], a[m], b[n]);
    }
}

// Software-pipelined variant for streaming weights: batches of U slices, the
// next batch's loads issued before the current batch's MFMAs.  The first
// batch's B (weight) loads are issued before `resolve_a` runs, so that a
// dependent gather of the A rows (token indices read from memory) overlaps
// the first weight fetch.
// With PIPE false the batches run one after the other (half the registers);
// only the first batch's weight loads still go out before `resolve_a`.
template <typename DT, int MB, int NB, int U, bool PIPE, typename ResolveA>
__device__ __forceinline__ void wave_gemm_stream(ResolveA resolve_a, const typename DT::storage *const (&b_rows)[NB],
                                                 int s0, int s1, f32x4 (&acc)[MB][NB])
{
    using S = typename DT::storage;
    const S *a_rows[MB];
    const int nfull = (s1 - s0) / U;
    Frag<DT> bc[U][NB], ac[U][MB];
    if (nfull > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int n = 0; n < NB; ++n) bc[u][n].load(b_rows[n] + (s0 + u) * 32);
    }
    resolve_a(a_rows);
    if (nfull > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MB; ++m) ac[u][m].load(a_rows[m] + (s0 + u) * 32);
    }
    int s = s0;
    if (!PIPE) {
        for (int it = 0; it < nfull; ++it, s += U) {
            if (it > 0) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int n = 0; n < NB; ++n) bc[u][n].load(b_rows[n] + (s + u) * 32);
#pragma unroll
                    for (int m = 0; m < MB; ++m) ac[u][m].load(a_rows[m] + (s + u) * 32);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int n = 0; n < NB; ++n) mma(acc[m][n], ac[u][m], bc[u][n]);
        }
    }
    for (int it = 0; PIPE && it < nfull; ++it, s += U) {
        Frag<DT> bn[U][NB], an[U][MB];
        const bool more = it + 1 < nfull;
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int n = 0; n < NB; ++n) bn[u][n].load(b_rows[n] + (s + U + u) * 32);
#pragma unroll
                for (int m = 0; m < MB; ++m) an[u][m].load(a_rows[m] + (s + U + u) * 32);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int n = 0; n < NB; ++n) mma(acc[m][n], ac[u][m], bc[u][n]);
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int n = 0; n < NB; ++n) bc[u][n] = bn[u][n];
#pragma unroll
                for (int m = 0; m < MB; ++m) ac[u][m] = an[u][m];
            }
        }
    }
    for (; s < s1; ++s) {
        Frag<DT> a[MB];
        Frag<DT> b[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) b[n].load(b_rows[n] + s * 32);
#pragma unroll
        for (int m = 0; m < MB; ++m) a[m].load(a_rows[m] + s * 32);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int n = 0; n < NB; ++n) mma(acc[m][n], a[m], b[n]);
    }
}

template <int MB, int NB>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MB][NB])
{
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Split-k reduction for a work-group of NW waves that computed the same tile
// over different k ranges: afterwards every wave holds the full sum, added in
// wave order (so the result does not depend on timing).
// red: LDS of NW * MB * NB * 256 floats.
template <int NW, int MB, int NB>
__device__ __forceinline__ void splitk_reduce(f32x4 (&acc)[MB][NB], float *red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    f32x4 *r4 = reinterpret_cast<f32x4 *>(red);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) r4[((wave * MB + m) * NB + n) * 64 + lane] = acc[m][n];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            f32x4 s = r4[((0 * MB + m) * NB + n) * 64 + lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                f32x4 v = r4[((w * MB + m) * NB + n) * 64 + lane];
                s[0] += v[0];
                s[1] += v[1];
                s[2] += v[2];
                s[3] += v[3];
            }
            acc[m][n] = s;
        }
}

template <int MB, int NB>
__device__ __forceinline__ void splitk_reduce4(f32x4 (&acc)[MB][NB], float *red)
{
    splitk_reduce<4, MB, NB>(acc, red);
}

}  // namespace flint
