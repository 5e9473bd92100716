// Shared device helpers for the Flint MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the others at their "no wait"
// maximum).  One in-order counter covers every vector-memory load and store
// of the wave.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Element tag types.  Storage of bf16 is uint16_t bit patterns.
struct BF16 {
    using storage = uint16_t;
    static constexpr int kBytes = 2;
};
struct F32 {
    using storage = float;
    static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t v)
{
    return __uint_as_float(((uint32_t)v) << 16);
}

// float32 -> bf16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// A 32-wide slice of the reduction dimension as one lane holds it for the
// 16x16 MFMA tiles: 8 consecutive elements.  For bf16 this is one
// v_mfma_f32_16x16x32_bf16 operand; for float32 it feeds eight
// v_mfma_f32_16x16x4_f32 steps.
template <typename DT> struct Frag;

template <> struct Frag<BF16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const bf16x8 *>(p); }
    __device__ __forceinline__ void zero()
    {
        u32x4 z = {0u, 0u, 0u, 0u};
        v = __builtin_bit_cast(bf16x8, z);
    }
};

template <> struct Frag<F32> {
    f32x4 lo, hi;
    __device__ __forceinline__ void load(const float *p)
    {
        lo = *reinterpret_cast<const f32x4 *>(p);
        hi = *reinterpret_cast<const f32x4 *>(p + 4);
    }
    __device__ __forceinline__ void zero()
    {
        lo = f32x4{0.f, 0.f, 0.f, 0.f};
        hi = lo;
    }
};

// acc(16x16, fp32) += A(16 x 32) * B(32 x 16) for one 32-wide k slice.
// Lane l holds A row (l & 15) and B column (l & 15), k elements 8*(l>>4)..+7.
// Output: lane l holds C[4*(l>>4) + i][l & 15], i = 0..3.
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<BF16> &a, const Frag<BF16> &b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<F32> &a, const Frag<F32> &b)
{
    // Eight k=4 steps; step j takes element j of each lane's 8, so step j covers
    // k = {j, 8+j, 16+j, 24+j} of the slice and the eight steps cover all 32.
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

template <typename DT> __device__ __forceinline__ void store_elem(typename DT::storage *p, float v);
template <> __device__ __forceinline__ void store_elem<BF16>(uint16_t *p, float v) { *p = f32_to_bf16(v); }
template <> __device__ __forceinline__ void store_elem<F32>(float *p, float v) { *p = v; }

template <typename DT> __device__ __forceinline__ float load_elem(const typename DT::storage *p);
template <> __device__ __forceinline__ float load_elem<BF16>(const uint16_t *p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_elem<F32>(const float *p) { return *p; }

// silu(g) * u in float32.
__device__ __forceinline__ float swiglu(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

}  // namespace flint
