// combine.hip -- Steps 4 and 5 of the expert-parallelism blog page (section
// 2.2): bring each expert output back to its token and form
//   out[t] = sum_k topk_w[t][k] * y[inv_pos[t][k]]  +  gate[t] * sum_j shared_y[j][t]
// On one GPU the return trip is a gather: y rows are read through inv_pos.
// Accumulation is fp32 in fixed k order (deterministic), rounded once to the
// output dtype.  Pairs computed on other GPUs (inv_pos = -1) are skipped, so a
// token with no local pair and no shared term gets exact zeros.
//
// One block per token with one thread per 8 consecutive features (up to
// 1024 threads: 896 for hidden 7168), so every y row of the token is read
// once with 16-byte loads; the token's local pairs are compacted in k order
// into LDS first.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T *p, float v[8]);
template <>
__device__ __forceinline__ void load8<f16>(const f16 *p, float v[8]) {
    const f16x8 x = *reinterpret_cast<const f16x8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)x[j];
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float v[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[j + 4] = b[j];
    }
}
template <typename T>
__device__ __forceinline__ void store8(T *p, const float v[8]);
template <>
__device__ __forceinline__ void store8<f16>(f16 *p, const float v[8]) {
    f16x8 x;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = to_f16(v[j]);
    *reinterpret_cast<f16x8 *>(p) = x;
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const float v[8]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

template <typename T>
__global__ __launch_bounds__(1024) void combine_kernel(CombineArgs a) {
    __shared__ int rows[16];
    __shared__ float gates[16];
    __shared__ int npairs;
    const int t = blockIdx.x;
    if (threadIdx.x == 0) {
        // local pairs of this token, compacted in k order
        int n = 0;
        for (int k = 0; k < a.K; ++k) {
            const int r = a.inv_pos[(size_t)t * a.K + k];
            if (r >= 0) {
                rows[n] = r;
                gates[n] = a.topk_w[(size_t)t * a.K + k];
                ++n;
            }
        }
        npairs = n;
    }
    __syncthreads();
    const int np = npairs;
    const T *y = reinterpret_cast<const T *>(a.y);
    const T *shy = reinterpret_cast<const T *>(a.shared_y);
    const bool sh = shy && a.n_shared > 0;
    const float gs = sh ? a.shared_gate[t] : 0.0f;
    T *out = reinterpret_cast<T *>(a.out) + (size_t)t * a.H;
    for (int i = threadIdx.x * 8; i < a.H; i += blockDim.x * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < np; ++q) {
            float v[8];
            load8<T>(y + (size_t)rows[q] * a.H + i, v);
            const float g = gates[q];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += g * v[j];
        }
        if (sh) {
            float sv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < a.n_shared; ++s) {
                float v[8];
                load8<T>(shy + ((size_t)s * a.T + t) * a.H + i, v);
#pragma unroll
                for (int j = 0; j < 8; ++j) sv[j] += v[j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += gs * sv[j];
        }
        store8<T>(out + i, acc);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    // one thread per 8 features, up to 1024 threads (whole waves)
    int threads = ((a.H / 8 + 63) / 64) * 64;
    if (threads > 1024) threads = 1024;
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL(combine_kernel<f16>, dim3(a.T), dim3(threads), 0, s, a);
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3(a.T), dim3(threads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
