// route_topk.hip -- softmax over all experts, top-K selection, shared gate.
//
// Step 1 of the expert-parallelism blog page (section 2.2) picks the K = 8
// highest-scoring experts of a token; Step 5 weights expert i's output by the
// softmax of the logits at i and the shared experts' output by a gate.
// Readings: the softmax runs over all E logits and the selected
// probabilities are not renormalised; ties go to the lower expert id; the
// shared gate is sigmoid(h . w_sg), whose logit the router GEMM writes as an
// extra column after the E expert columns.
//
// One wave per token.  Lane l holds logits e = l + 64*j (coalesced loads);
// each of the K rounds finds the wave-wide best (larger logit, then smaller
// id) with a butterfly of shuffles, so every lane agrees on the winner and
// the owning lane retires it.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// NS > 0: the number of K-slice partials, known at compile time (all loads
// issued up front, no branches); NS == 0: any count, runtime loop.
template <int EPL, int NS>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ parts, int nsplit,
                                                   size_t split_stride, int ld, int T, int E,
                                                   int K, int has_gate,
                                                   const float *__restrict__ bias,
                                                   int32_t *__restrict__ topk_idx,
                                                   float *__restrict__ topk_w,
                                                   float *__restrict__ shared_gate,
                                                   float *__restrict__ logits_out) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = lane_id();
    const float *l = parts + (size_t)t * ld;

    // logits = sum of the K-slice partials in slice order, then + bias
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        float acc = -INFINITY;
        if (e < E) {
            if (NS > 0) {
                float part[NS > 0 ? NS : 1];
#pragma unroll
                for (int zs = 0; zs < NS; ++zs) part[zs] = l[(size_t)zs * split_stride + e];
                acc = part[0];
#pragma unroll
                for (int zs = 1; zs < NS; ++zs) acc += part[zs];
            } else {
                acc = l[e];
                for (int zs = 1; zs < nsplit; ++zs) acc += l[(size_t)zs * split_stride + e];
            }
            if (bias) acc += bias[e];
        }
        v[j] = acc;
    }
    if (logits_out) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E) logits_out[(size_t)t * E + e] = v[j];
        }
    }

    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
        if (lane + 64 * j < E) z += expf(v[j] - m);
    z = wave_sum(z);

    uint32_t taken = 0;
    for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && e < bi))) {
                bv = v[j];
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, kWave);
            const int oi = __shfl_xor(bi, o, kWave);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == 0) {
            topk_idx[(size_t)t * K + k] = bi;
            topk_w[(size_t)t * K + k] = expf(bv - m) / z;
        }
    }
    if (has_gate && shared_gate && lane == 0) {
        float zg = l[E];
        for (int zs = 1; zs < nsplit; ++zs) zg += l[(size_t)zs * split_stride + E];
        shared_gate[t] = sigmoidf_(zg);
    }
}

template <int EPL>
hipError_t launch_e(dim3 grid, const float *logits, int nsplit, size_t split_stride, int ld,
                    int T, int E, int K, int has_gate, const float *bias, int32_t *topk_idx,
                    float *topk_w, float *shared_gate, float *logits_out, hipStream_t s) {
#define MOE_TOPK(NS)                                                                          \
    hipLaunchKernelGGL((topk_kernel<EPL, NS>), grid, dim3(256), 0, s, logits, nsplit,         \
                       split_stride, ld, T, E, K, has_gate, bias, topk_idx, topk_w,            \
                       shared_gate, logits_out)
    switch (nsplit) {  // the splits the router picks for common hidden sizes
    case 1: MOE_TOPK(1); break;
    case 2: MOE_TOPK(2); break;
    case 4: MOE_TOPK(4); break;
    case 7: MOE_TOPK(7); break;
    case 8: MOE_TOPK(8); break;
    case 14: MOE_TOPK(14); break;
    default: MOE_TOPK(0); break;
    }
#undef MOE_TOPK
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float *logits, int nsplit, size_t split_stride, int ld, int T,
                       int E, int K, int has_gate, const float *bias, int32_t *topk_idx,
                       float *topk_w, float *shared_gate, float *logits_out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    if (E <= 64)
        return launch_e<1>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    if (E <= 128)
        return launch_e<2>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    if (E <= 256)
        return launch_e<4>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    if (E <= 512)
        return launch_e<8>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    return launch_e<16>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, bias,
                        topk_idx, topk_w, shared_gate, logits_out, s);
}

}  // namespace moe
