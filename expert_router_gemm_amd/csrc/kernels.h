// kernels.h -- internal launch interface between moe_api.cpp and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- combine
// out[t] = sum over local k (k order) of topk_w[t][k] * y[inv_pos[t][k]]
//          + shared_gate[t] * sum_j shared_y[j][t]       (fp32 fma from 0)
struct CombineArgs {
    int T, K, H, n_shared, dtype;
    const void *y;
    const int32_t *inv_pos;
    const float *topk_w;
    const void *shared_y;   // [n_shared][T][H] or NULL
    const float *shared_gate;
    void *out;
    // Down projection with the combine fused (tiled kernel only): row ->
    // pair t*K + k, and one ticket per (token, 256-feature tile) holding the
    // token's local pair count (set by dispatch; taken to 0 by the GEMM).
    const int32_t *perm_src;
    int32_t *tickets;
};

// ---------------------------------------------------------------- GEMMs
enum : int { STREAM_STORE = 0, STREAM_SWIGLU = 1, STREAM_LOGITS = 2 };

struct StreamArgs {
    const void *x;          // [rows][K] activations (dtype, or fp8 codes)
    const float *x_scale;   // fp8 rows: per-row scale
    int x_broadcast;        // x row = r - group start (shared experts)
    const int32_t *gather;  // if set: x row = gather[r] / gather_div (perm_src / top_k)
    int gather_div;
    const int32_t *offsets; // [G+1] group row ranges, or NULL: uniform groups
    int rows_per_group;     // uniform groups: group g = rows [g*rpg, (g+1)*rpg)
    const void *w0;         // [G][N][K]: gate (SWIGLU) or the only matrix
    const void *w1;         // [G][N][K]: up (SWIGLU only)
    size_t w_group_stride;  // elements from one group's matrix to the next
    int w_frag;             // weights (w0, w1, w0b, w1b) in the fragment
                            // layout (see frag_offset), else row-major
    void *out;              // [rows][out_ld]
    int out_ld;
    int N, K;
    int ksplit;             // LOGITS only: K is split in ksplit equal slices;
    size_t split_stride;    // slice z writes out + z * split_stride (fp32)
    // Optional secondary groups (stream kernel only), placed before the
    // groups above in the grid: n_sec groups of rows2 rows each, weights
    // w0b/w1b [n_sec][N][K], output rows row2_base + g2*rows2 + i, input row
    // x2[i] (x2_broadcast) or x2[output row].  Lets the shared experts run in
    // the routed experts' launch.
    int n_sec;
    const void *x2;
    int x2_broadcast;
    const void *w0b, *w1b;
    int rows2, row2_base;
    // Down projection only (tiled kernel): with comb.out set, the launch
    // also forms the layer output from the rows it writes (see
    // gemm_tiled.hip); comb.y is not used (the rows are this launch's out).
    CombineArgs comb;
};

// Fragment layout of a [N][K] weight matrix (N a multiple of 16, K * esize
// a multiple of 64 bytes): 1 KB fragments, fragment (i, j) = rows 16i..16i+15
// x the 64 bytes of K from byte 64j, stored at byte (i * (K*esize/64) + j) *
// 1024; inside it, byte 256q + 16r + c is row 16i + r, row byte 64j + 16q +
// c.  Lane 16q + r of a wave thus reads one contiguous 1 KB per fragment --
// the MFMA operand layout (row r, K quarter q) that a row-major wave load
// gathers from 16 rows.  Byte offset of (row n, row byte b):
__host__ __device__ inline size_t frag_offset(size_t n, size_t b, size_t row_bytes) {
    return ((n >> 4) * (row_bytes >> 6) + (b >> 6)) * 1024 + ((b >> 4) & 3) * 256 +
           (n & 15) * 16 + (b & 15);
}

// dtype: DT_F16 / DT_F32 (weights and output); x_dtype: dtype or DT_FP8.
// Grid: ceil(N/64) x n_groups x zblocks; see gemm_stream.hip.
// est_rows: expected rows per group (host estimate), picks the kernel shape.
hipError_t launch_stream_gemm(const StreamArgs &a, int dtype, int x_dtype, int mode,
                              int n_groups, int zblocks, long est_rows, hipStream_t s);
// Whether launch_stream_gemm picks the same kernel (so the same summation
// order) for expected group sizes est_a and est_b.
bool stream_gemm_same_kernel(int dtype, int mode, long est_a, long est_b);

// LDS-tiled persistent variant for groups of many rows (fp16 only; K split
// for router logits).  max_tiles bounds the total 128-row tiles (sizes the
// grid).  Router logits use tiles of kTiledRouterRows rows.
constexpr int kTiledRouterRows = 128;
bool tiled_gemm_supported(const StreamArgs &a, int dtype, int x_dtype);
bool tiled_gemm_supported_shape(int K, int dtype, int x_dtype);
hipError_t launch_tiled_gemm(const StreamArgs &a, int mode, int n_groups, long max_tiles,
                             hipStream_t s);
// Sets up every tiled kernel on the current device (dynamic LDS limit,
// resident workgroup count), once per device; later calls return at once.
// Not a stream operation: the entry points call it before enqueueing, so
// their first call on a device sets the state that captured calls use.
hipError_t tiled_gemm_prepare();

// ---------------------------------------------------------------- routing
// Partial logits parts[z][T][ld] fp32, z < nsplit (E expert columns, then
// the shared-gate column if has_gate), summed in z order, plus bias ->
// topk_idx/topk_w [T][K], shared_gate [T], logits_out [T][E].  G > 0:
// group-limited selection (M of G groups), see moe_shape.n_groups.
hipError_t launch_topk(const float *parts, int nsplit, size_t split_stride, int ld, int T,
                       int E, int K, int has_gate, int G, int M, const float *bias,
                       int32_t *topk_idx,
                       float *topk_w, float *shared_gate, float *logits_out, hipStream_t s);

// ---------------------------------------------------------------- dispatch
struct DispatchArgs {
    int T, K, E, S, H;
    int dtype;              // of h
    int x_dtype;            // of x_perm (dtype or DT_FP8)
    const void *h;
    const int32_t *topk_idx;
    const int32_t *rep_off;
    const int32_t *rep_slot;
    uint64_t seed;
    void *x_perm;
    float *x_scale;
    int32_t *counts, *offsets, *perm_src, *inv_pos;
    // scratch
    int32_t *pair_code;     // [T*K]
    int32_t *chunk_counts;  // [C][S], C = ceil(T/64)
    // optional: tickets[t][f] = local pairs of token t, f < n_tiles (the
    // down projection's fused combine)
    int32_t *tickets;
    int n_tiles;
};
size_t dispatch_scratch_bytes(int T, int K, int S);
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s);

// ---------------------------------------------------------------- monitor
// counts[e] = #{p < pairs : topk_idx[p] == e}, e < E (E <= 1024).
hipError_t launch_expert_counts(const int32_t *topk_idx, long pairs, int E, int32_t *counts,
                                hipStream_t s);

// ---------------------------------------------------------------- combine
// The separate combine (CombineArgs above; perm_src and tickets unused).
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);

// ---------------------------------------------------------------- layout
// dst[m] = fragment layout of the row-major src[m] ([rows][row_bytes]),
// m < n_mats (rows % 16 == 0, row_bytes % 64 == 0, no overlap).
hipError_t launch_pack_frag(const void *src, void *dst, long n_mats, int rows, int row_bytes,
                            hipStream_t s);

}  // namespace moe
