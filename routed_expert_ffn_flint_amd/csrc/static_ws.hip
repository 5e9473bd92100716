// flint_moe_forward_static: the whole layer with its scratch in a file-scope
// device array instead of a caller-provided workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array `scratch` holds kStaticScratchBytes on every GPU the library runs
// on, for as long as the process lives.  Host code never passes its name to a
// kernel (in host code it is a host-side stand-in, not a device address): at
// the first call on a device, with that device current, hipGetSymbolAddress
// gives that device's copy, and the address is kept per device.  Every call on
// one GPU shares that GPU's array; the layer clears what must start at zero
// with fill kernels, so earlier contents do not matter, but calls that overlap
// on one GPU (different streams, different threads) race on it.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/flint_moe.h"

namespace flint {
// abi.cpp: every check flint_moe_forward makes except the workspace's.
flint_status check_forward_call(const flint_moe_dims *d, int32_t T, const void *x, const flint_moe_weights *wt,
                                void *out, flint_dtype out_dtype, int32_t *topk_idx_out, float *topk_w_out);
}  // namespace flint

namespace {

constexpr size_t kStaticScratchBytes = FLINT_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// This device's copy of `scratch`, looked up once per device.  Returns
// nullptr (and the status to report) if the device or the lookup fails.
void *scratch_address(flint_status *st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = FLINT_DEVICE_ERROR;
        return nullptr;
    }
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
        *st = FLINT_DEVICE_ERROR;
        return nullptr;
    }
    g_scratch_addr[dev].store(addr, std::memory_order_release);
    return addr;
}

}  // namespace

extern "C" flint_status flint_moe_forward_static(const flint_moe_dims *d, int32_t T, const void *x,
                                                 const flint_moe_weights *weights, void *out,
                                                 flint_dtype out_dtype, int32_t *topk_idx_out,
                                                 float *topk_w_out, void *stream)
{
    // argument errors first, with the codes flint_moe_forward gives them, then
    // the size limit: all on the host, before the device is touched
    flint_status st = flint::check_forward_call(d, T, x, weights, out, out_dtype, topk_idx_out, topk_w_out);
    if (st != FLINT_OK || T == 0) return st;
    if (flint_moe_workspace_bytes(d, T) > kStaticScratchBytes) return FLINT_WORKSPACE_TOO_SMALL;
    void *ws = scratch_address(&st);
    if (!ws) return st;
    return flint_moe_forward(d, T, x, weights, out, out_dtype, topk_idx_out, topk_w_out, ws, kStaticScratchBytes,
                             stream);
}
