// Work-group scheduling and wait helpers of the LDS-staged expert products
// (tiled.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace flint {
namespace {

constexpr int kXcds = 8;
constexpr int kRowGroup = 8;  // row tiles per group of shared-weight items

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// Item of this work-group, or -1.  Work-groups are dealt to the XCDs
// round-robin (blockIdx.x % 8 is the XCD); XCD j runs the j-th eighth of the
// items, in order, so items next to each other in the order (the n-tiles of
// one expert tile, which gather the same rows; consecutive tiles of one
// expert, which read the same weights) share that XCD's L2.  The grid is sized
// for the most items the routing can produce.
__device__ __forceinline__ int xcd_item(int total)
{
    const int per = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    const int item = (blockIdx.x % kXcds) * per + slot;
    return (slot < per && item < total) ? item : -1;
}

// The same for a launch of ns shared-weight items followed by nr routed ones:
// each XCD takes an eighth of each kind (shared items first), so a kind whose
// items are longer (a wider shared expert) loads every XCD alike (T = 16384
// down product: 604 -> 481 us).  The grid holds 8 * (ceil(ns / 8) +
// ceil(routed capacity / 8)) work-groups.
__device__ __forceinline__ int xcd_item2(int ns, int nr)
{
    const int ps = (ns + kXcds - 1) / kXcds, pr = (nr + kXcds - 1) / kXcds;
    const int x = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    if (slot < ps) {
        const int item = x * ps + slot;
        return item < ns ? item : -1;
    }
    const int s2 = slot - ps;
    const int r = x * pr + s2;
    return (s2 < pr && r < nr) ? ns + r : -1;
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace
}  // namespace flint
