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
// One wave per token.  Lane l holds logits e = l + 64*j (coalesced loads).
// Each of the K selection rounds is one wave-wide maximum of a 64-bit key
// (order-preserving bits of the logit above the complement of the id, so a
// larger logit wins and equal logits go to the smaller id), reduced with DPP
// row shifts and row broadcasts into lane 63 and read back as a scalar; the
// owning lane retires the winner.  Lane k keeps the k-th selection, so the
// K indices and gates leave in one coalesced store each.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// One DPP step of a wave-wide maximum: this lane's key against the key of
// the lane CTRL names (lanes with no source, or masked off, keep their own).
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ void dpp_max_step(uint32_t &hi, uint32_t &lo) {
    const uint32_t oh = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, BANK_MASK, false);
    const uint32_t ol = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, BANK_MASK, false);
    const bool gt = oh > hi || (oh == hi && ol > lo);
    hi = gt ? oh : hi;
    lo = gt ? ol : lo;
}

// Wave-wide maximum of the 64-bit key (hi, lo), returned in every lane:
// row_shr 1, 2, 4, 8 leave each 16-lane row's maximum in its lane 15,
// row_bcast 15 and 31 carry it across rows into lane 63.
__device__ __forceinline__ void wave_max_key(uint32_t &hi, uint32_t &lo) {
    dpp_max_step<0x111, 0xf, 0xf>(hi, lo);  // row_shr:1
    dpp_max_step<0x112, 0xf, 0xf>(hi, lo);  // row_shr:2
    dpp_max_step<0x114, 0xf, 0xf>(hi, lo);  // row_shr:4
    dpp_max_step<0x118, 0xf, 0xf>(hi, lo);  // row_shr:8
    dpp_max_step<0x142, 0xa, 0xf>(hi, lo);  // row_bcast:15 into rows 1, 3
    dpp_max_step<0x143, 0xc, 0xf>(hi, lo);  // row_bcast:31 into rows 2, 3
    hi = __builtin_amdgcn_readlane(hi, 63);
    lo = __builtin_amdgcn_readlane(lo, 63);
}

// Order-preserving map of a finite float to uint32 (-0 and +0 map alike).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    const uint32_t b = v == 0.0f ? 0u : __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// NS > 0: the number of K-slice partials, known at compile time (all loads
// issued up front, no branches); NS == 0: any count, runtime loop.
template <int EPL, int NS>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ parts, int nsplit,
                                                   size_t split_stride, int ld, int T, int E,
                                                   int K, int has_gate, int G, int M,
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

    // Group-limited routing (G > 0): G contiguous groups of E/G experts; a
    // group's score is its best logit; the M best groups (ties: lower group
    // id) stay eligible.  Lane g ends up holding group g's key.
    uint32_t allowed = 0xffffffffu;  // bit j: expert lane + 64 j is eligible
    if (G > 0) {
        const int gs = E / G;
        uint32_t g_hi = 0, g_lo = 0;
        for (int g = 0; g < G; ++g) {
            uint32_t hi = 0, lo = 0;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane + 64 * j;
                if (e < E && e / gs == g) hi = max(hi, ordered_bits(v[j]));
            }
            wave_max_key(hi, lo);
            if (lane == g) {
                g_hi = hi;
                g_lo = ~(uint32_t)g;
            }
        }
        uint64_t keep = 0;
        for (int r = 0; r < M; ++r) {
            uint32_t hi = g_hi, lo = g_lo;
            wave_max_key(hi, lo);
            const int bg = (int)~lo;
            keep |= 1ull << bg;
            if (lane == bg) g_hi = g_lo = 0;
        }
        allowed = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && ((keep >> (e / gs)) & 1ull)) allowed |= 1u << j;
        }
    }

    // K rounds; round 0 yields the maximum logit m.  Keys of absent experts
    // and of experts already taken or not eligible are 0, below every
    // finite logit's key.
    uint32_t taken = ~allowed;
    int my_id = 0;
    float my_v = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint32_t hi = 0, lo = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((taken >> j) & 1u)) {
                const uint32_t h = ordered_bits(v[j]), l = ~(uint32_t)e;
                if (h > hi || (h == hi && l > lo)) {
                    hi = h;
                    lo = l;
                }
            }
        }
        wave_max_key(hi, lo);
        const int bi = (int)~lo;
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == k) {
            my_id = bi;
            my_v = from_ordered_bits(hi);
        }
    }
    const float m = __shfl(my_v, 0, kWave);
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
        if (lane + 64 * j < E) z += expf(v[j] - m);
    z = wave_sum(z);
    if (lane < K) {
        topk_idx[(size_t)t * K + lane] = my_id;
        topk_w[(size_t)t * K + lane] = expf(my_v - m) / z;
    }
    if (has_gate && shared_gate && lane == 0) {
        // the gate column's partials, summed in slice order like the logits
        // (all loads issued before the first add when NS is known)
        float zg;
        if (NS > 0) {
            float part[NS > 0 ? NS : 1];
#pragma unroll
            for (int zs = 0; zs < NS; ++zs) part[zs] = l[(size_t)zs * split_stride + E];
            zg = part[0];
#pragma unroll
            for (int zs = 1; zs < NS; ++zs) zg += part[zs];
        } else {
            zg = l[E];
            for (int zs = 1; zs < nsplit; ++zs) zg += l[(size_t)zs * split_stride + E];
        }
        shared_gate[t] = sigmoidf_(zg);
    }
}

template <int EPL>
hipError_t launch_e(dim3 grid, const float *logits, int nsplit, size_t split_stride, int ld,
                    int T, int E, int K, int has_gate, int G, int M, const float *bias,
                    int32_t *topk_idx,
                    float *topk_w, float *shared_gate, float *logits_out, hipStream_t s) {
#define MOE_TOPK(NS)                                                                          \
    hipLaunchKernelGGL((topk_kernel<EPL, NS>), grid, dim3(256), 0, s, logits, nsplit,         \
                       split_stride, ld, T, E, K, has_gate, G, M, bias, topk_idx, topk_w,      \
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
                       int E, int K, int has_gate, int G, int M, const float *bias,
                       int32_t *topk_idx,
                       float *topk_w, float *shared_gate, float *logits_out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    if (E <= 64)
        return launch_e<1>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, G, M, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    if (E <= 128)
        return launch_e<2>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, G, M, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    if (E <= 256)
        return launch_e<4>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, G, M, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    if (E <= 512)
        return launch_e<8>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, G, M, bias,
                           topk_idx, topk_w, shared_gate, logits_out, s);
    return launch_e<16>(grid, logits, nsplit, split_stride, ld, T, E, K, has_gate, G, M, bias,
                        topk_idx, topk_w, shared_gate, logits_out, s);
}

}  // namespace moe
