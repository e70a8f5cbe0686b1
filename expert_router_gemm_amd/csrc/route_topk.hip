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

template <int EPL>
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
            // issue every slice's load before summing (at most 16 slices)
            float part[16];
#pragma unroll
            for (int zs = 0; zs < 16; ++zs)
                part[zs] = zs < nsplit ? l[(size_t)zs * split_stride + e] : 0.0f;
            acc = part[0];
#pragma unroll
            for (int zs = 1; zs < 16; ++zs)
                if (zs < nsplit) acc += part[zs];
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

}  // namespace

hipError_t launch_topk(const float *logits, int nsplit, size_t split_stride, int ld, int T,
                       int E, int K, int has_gate, const float *bias, int32_t *topk_idx,
                       float *topk_w, float *shared_gate, float *logits_out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4), block(256);
    if (E <= 64)
        hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, nsplit, split_stride, ld, T,
                           E, K, has_gate, bias, topk_idx, topk_w, shared_gate, logits_out);
    else if (E <= 128)
        hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, logits, nsplit, split_stride, ld, T,
                           E, K, has_gate, bias, topk_idx, topk_w, shared_gate, logits_out);
    else if (E <= 256)
        hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, nsplit, split_stride, ld, T,
                           E, K, has_gate, bias, topk_idx, topk_w, shared_gate, logits_out);
    else if (E <= 512)
        hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, logits, nsplit, split_stride, ld, T,
                           E, K, has_gate, bias, topk_idx, topk_w, shared_gate, logits_out);
    else
        hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, logits, nsplit, split_stride, ld, T,
                           E, K, has_gate, bias, topk_idx, topk_w, shared_gate, logits_out);
    return hipGetLastError();
}

}  // namespace moe
