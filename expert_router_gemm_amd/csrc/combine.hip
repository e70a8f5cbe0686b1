// combine.hip -- Steps 4 and 5 of the expert-parallelism blog page (section
// 2.2): bring each expert output back to its token and form
//   out[t] = sum_k topk_w[t][k] * y[inv_pos[t][k]]  +  gate[t] * sum_j shared_y[j][t]
// On one GPU the return trip is a gather: y rows are read through inv_pos.
// Accumulation is fp32 in fixed k order (deterministic), rounded once to the
// output dtype: acc = fma(w_k, y_k, acc) from 0 over the local pairs, then
// acc = fma(gate, sum of shared rows, acc).  The down projection's fused
// combine (gemm_tiled.hip) uses the same sequence, so both give the same bits.  Pairs computed on other GPUs (inv_pos = -1) are skipped, so a
// token with no local pair and no shared term gets exact zeros.
//
// One block per token with one thread per 8 consecutive features (up to
// 1024 threads: 896 for hidden 7168; per two chunks of 8 for large batches),
// so every y row of the token is read once with 16-byte loads; the token's local pairs are compacted in k order
// into LDS first (one wave, a ballot and popcounts), and each thread loads
// them 4 at a time.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// 16 bytes of a row: 8 fp16 values, or two 16-byte halves of 8 fp32 values
template <typename T>
struct Raw8;
template <>
struct Raw8<f16> {
    f16x8 v;
    __device__ __forceinline__ void load(const f16 *p) { v = *reinterpret_cast<const f16x8 *>(p); }
    __device__ __forceinline__ float operator[](int j) const { return (float)v[j]; }
};
template <>
struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const f32x4 *>(p);
        b = *reinterpret_cast<const f32x4 *>(p + 4);
    }
    __device__ __forceinline__ float operator[](int j) const { return j < 4 ? a[j] : b[j - 4]; }
};

template <typename T>
__device__ __forceinline__ void store8(T *p, const float v[8]);
template <>
__device__ __forceinline__ void store8<f16>(f16 *p, const float v[8]) {
    // 8 fp32 sums -> fp16 as one vector: v_cvt_pk_f16_f32 (round to
    // nearest even), the rounding the fused tail in gemm_tiled.hip writes
    // out explicitly (plain asm here costs the kernel ~2 us of branches)
    f32x8 w;
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = v[j];
    *reinterpret_cast<f16x8 *>(p) = __builtin_convertvector(w, f16x8);
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const float v[8]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Rows are summed in batches of 4 whose loads are in flight together (one
// round trip per 4 rows instead of per row, at 4 fp16 vectors of registers).
constexpr int kMaxPairs = 16;  // top-K limit of the shape check
constexpr int kCombineTwoChunkT = 2048;  // tokens from which a thread sums two chunks

template <typename T, int CH>
__global__ __launch_bounds__(1024) void combine_kernel(CombineArgs a) {
    __shared__ int rows[kMaxPairs];
    __shared__ float gates[kMaxPairs];
    __shared__ int npairs;
    const int t = blockIdx.x;
    if (threadIdx.x < 64) {
        // the token's local pairs, compacted in k order: lane k reads pair k,
        // its slot among the local pairs is the count of local lanes below it
        const int k = threadIdx.x;
        int r = -1;
        float g = 0.0f;
        if (k < a.K) {
            r = a.inv_pos[(size_t)t * a.K + k];
            g = a.topk_w[(size_t)t * a.K + k];
        }
        const uint64_t local = __ballot(r >= 0);
        if (r >= 0) {
            const int pos = __popcll(local & ((1ull << k) - 1));
            rows[pos] = r;
            gates[pos] = g;
        }
        if (k == 0) npairs = __popcll(local);
    }
    __syncthreads();
    const int np = npairs;
    const T *y = reinterpret_cast<const T *>(a.y);
    const T *shy = reinterpret_cast<const T *>(a.shared_y);
    const bool sh = shy && a.n_shared > 0;
    const float gs = sh ? a.shared_gate[t] : 0.0f;
    T *out = reinterpret_cast<T *>(a.out) + (size_t)t * a.H;
    for (int i0 = threadIdx.x * 8; i0 < a.H; i0 += blockDim.x * 8 * CH) {
        float acc[CH][8];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[c][j] = 0.f;
        // batches of 4 rows x CH chunks: their loads are in flight together
        for (int q0 = 0; q0 < np; q0 += 4) {
            Raw8<T> v[4][CH];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int i = i0 + c * blockDim.x * 8;
                    if (q0 + q < np && i < a.H) v[q][c].load(y + (size_t)rows[q0 + q] * a.H + i);
                }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q0 + q < np) {
                    const float g = gates[q0 + q];
#pragma unroll
                    for (int c = 0; c < CH; ++c)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            acc[c][j] = __builtin_fmaf(g, v[q][c][j], acc[c][j]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = i0 + c * blockDim.x * 8;
            if (i >= a.H) continue;
            if (sh) {
                float sv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                for (int s = 0; s < a.n_shared; ++s) {
                    Raw8<T> u;
                    u.load(shy + ((size_t)s * a.T + t) * a.H + i);
#pragma unroll
                    for (int j = 0; j < 8; ++j) sv[j] += u[j];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[c][j] = __builtin_fmaf(gs, sv[j], acc[c][j]);
            }
            store8<T>(out + i, acc[c]);
        }
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    // one thread per 8 features, up to 1024 threads (whole waves)
    if (a.K < 1 || a.K > kMaxPairs) return hipErrorInvalidValue;
    // Batches of thousands of tokens: two chunks of 8 features per thread
    // (their loads in flight together, half-size blocks, twice the blocks
    // per CU): prefill combine 86 -> 72 us at T = 16384.  Decode batches keep
    // one chunk per thread (more waves for few tokens).  Same sums either way.
    const bool two = a.T >= kCombineTwoChunkT;
    int threads = ((a.H / (two ? 16 : 8) + 63) / 64) * 64;
    if (threads > 1024) threads = 1024;
    if (a.dtype == DT_F16) {
        if (two)
            hipLaunchKernelGGL((combine_kernel<f16, 2>), dim3(a.T), dim3(threads), 0, s, a);
        else
            hipLaunchKernelGGL((combine_kernel<f16, 1>), dim3(a.T), dim3(threads), 0, s, a);
    } else {
        if (two)
            hipLaunchKernelGGL((combine_kernel<float, 2>), dim3(a.T), dim3(threads), 0, s, a);
        else
            hipLaunchKernelGGL((combine_kernel<float, 1>), dim3(a.T), dim3(threads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace moe
