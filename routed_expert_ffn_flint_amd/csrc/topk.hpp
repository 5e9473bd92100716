// Per-token routing arithmetic shared by the top-k kernels (route.hip) and the
// fused decode kernel (fused.hip): the float32 sigmoid score, the normalised
// weight and the one-wave top-K selection.
//
// Serving-kit review, "The architecture, from the config": sigmoid router
// scores, the top-k of them renormalised (not a softmax); 6 of 256 experts.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace flint {

// sigmoid(z) in float32.  For z < 0 it is e^z / (1 + e^z): 1 / (1 + e^-z)
// would overflow e^-z to infinity below z = -88.7 and return 0, where the
// score is still a float32 subnormal (it reaches 0 only below about -103.3).
__device__ __forceinline__ float score_from_logit(float z)
{
    if (z < 0.0f) {
        const float e = expf(z);
        return e / (1.0f + e);
    }
    return 1.0f / (1.0f + expf(-z));
}

// Routing weight of a selected expert: score / sum of the selected scores,
// the sum in double.  When every selected score is zero (every logit below
// about -103.3) the quotient is 0/0; each expert then gets 1/K, the share
// equal scores get.
__device__ __forceinline__ float routing_weight(float s, double sum, int K)
{
    return sum > 0.0 ? (float)((double)s / sum) : (float)(1.0 / K);
}

// Top-K of one token by one wave (E <= 256: four candidates per lane, expert
// lane + 64*i), by a bitwise search for the K-th largest score: float32 scores
// are >= 0, so their bit patterns order like the values, and the K-th largest
// pattern is the largest v with at least K patterns >= v, found one bit at a
// time from the top with wave-wide counts (ballots).  Then every score above
// it is selected, and of those equal to it the lowest expert indices up to K
// (with an early stop, the prefix found instead: see below).
// A chain of ~32 short compare/count steps instead of log2(64) merges of
// sorted 8-entry lists.  Lane k < K gets the k-th selected expert (ascending
// ids) and its weight (s over the sum of the K selected, the sum in double in
// ascending id order).  ls, le: K floats and K ints of LDS for this wave.
__device__ __forceinline__ void wave_topk_select(const float *zt, size_t split_stride, int nsplit, int E, int K,
                                                 float *ls, int *le, int &idx_out, float &w_out)
{
    const int lane = threadIdx.x & 63;
    uint32_t u[4];
    bool v[4];
    float z[4];
    // every load unconditional (experts past E read expert 0 and are masked),
    // so the four go out together instead of one latency each
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E;
        z[i] = zt[v[i] ? e : 0];
    }
    for (int sp = 1; sp < nsplit; ++sp)  // partial sums, in order
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] += zt[sp * split_stride + (v[i] ? lane + 64 * i : 0)];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = v[i] ? __float_as_uint(score_from_logit(z[i])) : 0u;
    // (bit 31, the sign, is 0 in every score.)  Once exactly K patterns are
    // >= the prefix, those K are the selection: the loop stops there (the
    // count is wave-uniform), typically after half the bits.
    uint32_t thr = 0;
    for (int bit = 30; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(v[i] && u[i] >= cand));
        if (cnt >= K) {
            thr = cand;
            if (cnt == K) break;
        }
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) gt += __popcll(__ballot(v[i] && u[i] > thr));
    const int need = K - gt;  // taken from the scores equal to thr, lowest ids first
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint64_t eq = __ballot(v[i] && u[i] == thr);
        const int eq_rank = eq_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
        const bool sel = v[i] && (u[i] > thr || (u[i] == thr && eq_rank < need));
        const uint64_t sm = __ballot(sel);
        if (sel) {
            const int r = sel_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
            ls[r] = __uint_as_float(u[i]);
            le[r] = lane + 64 * i;
        }
        eq_before += __popcll(eq);
        sel_before += __popcll(sm);
    }
    __builtin_amdgcn_wave_barrier();
    double sum = 0.0;
    for (int k = 0; k < K; ++k) sum += (double)ls[k];
    idx_out = lane < K ? le[lane] : 0;
    w_out = lane < K ? routing_weight(ls[lane], sum, K) : 0.0f;
}

}  // namespace flint
