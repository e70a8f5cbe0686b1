// expert_counts.hip -- per-expert token counts of one forward, the monitor
// input of the load balancer (expert-parallelism blog page, section 6.2:
// count each expert's arrivals).  One launch clears the counts, a second
// one builds a histogram per block in LDS and adds it to the global counts;
// integer adds, so the result does not depend on their order.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void counts_clear_kernel(int32_t *counts, int E) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < E) counts[i] = 0;
}

__global__ __launch_bounds__(256) void counts_kernel(const int32_t *__restrict__ idx, long n,
                                                     int E, int32_t *__restrict__ counts) {
    __shared__ int32_t h[1024];
    for (int i = threadIdx.x; i < E; i += 256) h[i] = 0;
    __syncthreads();
    for (long p = (long)blockIdx.x * 256 + threadIdx.x; p < n; p += (long)gridDim.x * 256) {
        const int e = idx[p];
        if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += 256)
        if (h[i]) atomicAdd(&counts[i], h[i]);
}

}  // namespace

hipError_t launch_expert_counts(const int32_t *topk_idx, long pairs, int E, int32_t *counts,
                                hipStream_t s) {
    hipLaunchKernelGGL(counts_clear_kernel, dim3((E + 255) / 256), dim3(256), 0, s, counts, E);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pairs <= 0) return e;
    long blocks = (pairs + 255) / 256;
    if (blocks > 256) blocks = 256;
    hipLaunchKernelGGL(counts_kernel, dim3((unsigned)blocks), dim3(256), 0, s, topk_idx, pairs,
                       E, counts);
    return hipGetLastError();
}

}  // namespace moe
