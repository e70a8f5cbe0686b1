// noalloc.hip -- moe_layer_forward_noalloc: the whole layer (Steps 1-5 of
// the expert-parallelism blog page, section 2.2) for callers that cannot
// allocate device memory -- code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc.  The layer's workspace (router
// partials, routing, dispatch indices, hm and y rows, dispatch scratch) is
// a static device array of this library instead of a caller buffer; the
// caller still passes inputs, weights and the output.
//
// The array lives once per device for the life of the process.  In host
// code its name is only a host-side stand-in, so the device address is
// looked up with hipGetSymbolAddress on the first call on each device (with
// that device current) and kept per device; kernels only ever receive that
// address.  Every call on a device shares the array: calls that overlap on
// one GPU (two streams, or two host threads without ordering) race on it.
// No kernel of the layer reads workspace memory it has not written in the
// same call, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/moe.h"
#include "api_internal.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Device address of `scratch` on each device, 0 until the first call there.
std::atomic<void *> g_scratch[kMaxDevices];

moe_status scratch_of_current_device(void **p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MOE_ERR_NO_DEVICE;
    void *q = g_scratch[dev].load(std::memory_order_acquire);
    if (!q) {
        // a race between two first calls repeats the lookup; both store the
        // same address
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
            return MOE_ERR_NO_DEVICE;
        g_scratch[dev].store(q, std::memory_order_release);
    }
    *p = q;
    return MOE_OK;
}

}  // namespace

MOE_EXPORT moe_status moe_layer_forward_noalloc(const moe_shape *shape, const moe_weights *w,
                                                const moe_slot_map *map, int32_t T,
                                                const void *h, void *out, void *stream) {
    moe_status st = moe::layer_forward_validate(shape, w, map, T, h, out);
    if (st != MOE_OK || T == 0) return st;
    if (moe_workspace_bytes(shape, T) > kScratchBytes) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != MOE_OK) return st;
    return moe::layer_forward_run(shape, w, map, T, h, out, ws, kScratchBytes, nullptr, stream);
}
