// probe_read.hip -- HBM read-rate probe for the benchmark's reference record
// (libmoe_probe.so; not part of libmoe or its C ABI in include/moe.h).
//
// The decode expert GEMMs are weight streams: each wave reads contiguous
// 1 KB pieces with nontemporal 16-byte loads.  This kernel does only that,
// so its best rate over a few launch shapes is the read rate such a stream
// can reach on this GPU, the measured counterpart of the 8 TB/s published
// peak.  Block b reads slabs b, b + grid, ... of `slab` bytes each; wave w
// of a block reads pieces w, w + 4, ... of the slab, `unroll` pieces in
// flight; each thread folds what it read into one word (so nothing is
// optimised away) and stores it to out[global thread id].
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_slabs_kernel(const u32x4 *p, size_t slab16, size_t nslab,
                                                         uint32_t *out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t acc = 0;
    const size_t pieces = slab16 / 64;  // 1 KB pieces per slab
    for (size_t s = blockIdx.x; s < nslab; s += gridDim.x) {
        const u32x4 *q = p + s * slab16;
        size_t k = wave;
        for (; k + 4 * (U - 1) < pieces; k += 4 * U) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(q + (k + 4 * u) * 64 + lane);
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= v[u][0] + v[u][1] + v[u][2] + v[u][3];
        }
        for (; k < pieces; k += 4) acc ^= q[k * 64 + lane][0];
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

// Reads `bytes` at `buf` once on `stream` (NULL: the default stream).
// bytes and slab: multiples of 1024, slab divides bytes; blocks >= 1;
// unroll 4 or 8; out: blocks * 256 uint32 words.  Returns 0, or -1 on a
// bad argument (nothing launched), or the HIP error of the launch.
extern "C" __attribute__((visibility("default"))) int moe_probe_read(const void *buf, size_t bytes,
                                                                     size_t slab, int blocks,
                                                                     int unroll, uint32_t *out,
                                                                     void *stream) {
    if (!buf || !out || blocks < 1 || slab < 1024 || slab % 1024 || bytes % slab ||
        (unroll != 4 && unroll != 8))
        return -1;
    const u32x4 *p = static_cast<const u32x4 *>(buf);
    const size_t slab16 = slab / 16, nslab = bytes / slab;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (unroll == 4)
        hipLaunchKernelGGL(read_slabs_kernel<4>, dim3(blocks), dim3(256), 0, s, p, slab16, nslab, out);
    else
        hipLaunchKernelGGL(read_slabs_kernel<8>, dim3(blocks), dim3(256), 0, s, p, slab16, nslab, out);
    return (int)hipGetLastError();
}
