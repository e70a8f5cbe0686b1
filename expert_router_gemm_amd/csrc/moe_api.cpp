// moe_api.cpp -- the C ABI declared in include/moe.h: host-side validation,
// workspace layout and the launch sequence of the layer.  No allocation, no
// synchronisation, no global state.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"
#include "api_internal.h"
#include "kernels.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace moe;

constexpr int kMaxExperts = 1024;
constexpr int kMaxSlots = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxShared = 16;
constexpr int kMaxGroupsRoute = 64;  // expert groups of group-limited routing
constexpr int64_t kMaxTokens = 1 << 20;
// hidden and inter: the LDS-tiled GEMM forms a tile's byte ranges and row
// offsets (up to 256 rows of K fp16 values) in 32 bits
constexpr int kMaxDim = 65536;
// moe_pack_weights: matrices per call (a whole layer's gate, up or down
// weights, replicas included, is at most a few thousand).
constexpr int64_t kMaxPackMats = 1 << 20;

inline size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline int act_bytes(const moe_shape &s) { return s.act == MOE_F32 ? 4 : 2; }
inline int has_gate(const moe_shape &s) { return (s.flags & MOE_F_SHARED) ? 1 : 0; }

constexpr int kRouterMaxSplit = 16;      // largest router K split
constexpr int kRouterTiledMinT = 2048;   // smallest batch on the LDS-tiled router

// Router plan.  Large batches (T >= 2048, fp16) use the LDS-tiled kernel
// and small ones the weight-stream kernel; either way K is split (slices a
// multiple of the kernel's K granularity, at most kRouterMaxSplit) so
// that the workgroup count comes closest to 256.  The top-K kernel sums the
// slices in order.
struct RouterPlan {
    bool tiled;
    int ksplit;
};

RouterPlan router_plan(const moe_shape &s, int T) {
    const int N = s.n_experts + has_gate(s);
    RouterPlan p;
    p.tiled = T >= kRouterTiledMinT && tiled_gemm_supported_shape(s.hidden, s.act, s.act);
    const int tr = kTiledRouterRows;
    const long base = p.tiled ? (long)((N + 255) / 256) * ((T + tr - 1) / tr)
                              : (long)((N + 63) / 64) * ((T + 63) / 64);
    // fp16 stream path: K slices that are multiples of 512 let the 4 waves of
    // a block split each slice (see launch_stream_gemm); other sizes fall
    // back to the 128 granularity of one wave per slice
    int gran = p.tiled ? 128 : 4 * (s.act == MOE_F32 ? 16 : 32);
    if (!p.tiled && s.act != MOE_F32 && s.hidden % 512 == 0) gran = 512;
    // the valid split whose workgroup count is closest to 256 (measured:
    // 224 blocks beat 112 and 448 at decode sizes)
    p.ksplit = 1;
    long best = -1;
    for (int d = 1; d <= kRouterMaxSplit; ++d) {
        if (s.hidden % (d * gran)) continue;
        const long dist = base * d > 256 ? base * d - 256 : 256 - base * d;
        if (best < 0 || dist < best) {
            best = dist;
            p.ksplit = d;
        }
    }
    return p;
}

int router_ksplit(const moe_shape &s, int T) { return router_plan(s, T).ksplit; }

size_t route_ws_bytes(const moe_shape &s, int T) {
    return up256((size_t)router_ksplit(s, T) * T * (s.n_experts + has_gate(s)) * 4);
}

moe_status check_shape(const moe_shape *s) {
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->flags & ~(MOE_F_SHARED | MOE_F_FUSED_COMBINE)) return MOE_ERR_INVALID_ARG;
    if (s->w_layout != MOE_W_ROWMAJOR && s->w_layout != MOE_W_FRAG) return MOE_ERR_INVALID_ARG;
    if (s->hidden <= 0 || s->inter <= 0 || s->hidden % 128 || s->inter % 128) return MOE_ERR_SHAPE;
    if (s->hidden > kMaxDim || s->inter > kMaxDim) return MOE_ERR_SHAPE;
    if (s->n_experts < 1 || s->n_experts > kMaxExperts) return MOE_ERR_SHAPE;
    if (s->top_k < 1 || s->top_k > kMaxTopK || s->top_k > s->n_experts) return MOE_ERR_SHAPE;
    if (s->n_slots < 1 || s->n_slots > kMaxSlots) return MOE_ERR_SHAPE;
    if (s->n_shared < 0 || s->n_shared > kMaxShared) return MOE_ERR_SHAPE;
    if ((s->flags & MOE_F_SHARED) && s->n_shared < 1) return MOE_ERR_SHAPE;
    if (s->act != MOE_F32 && s->act != MOE_F16) return MOE_ERR_DTYPE;
    if (s->dispatch != s->act && !(s->dispatch == MOE_FP8_E4M3 && s->act == MOE_F16)) return MOE_ERR_DTYPE;
    if (s->n_groups != 0) {
        if (s->n_groups < 0 || s->n_groups > kMaxGroupsRoute || s->n_experts % s->n_groups)
            return MOE_ERR_SHAPE;
        if (s->topk_groups < 1 || s->topk_groups > s->n_groups) return MOE_ERR_SHAPE;
        if ((long)s->top_k > (long)s->topk_groups * (s->n_experts / s->n_groups)) return MOE_ERR_SHAPE;
    } else if (s->topk_groups != 0) {
        return MOE_ERR_SHAPE;
    }
    return MOE_OK;
}

moe_status check_T(int32_t T) { return (T < 0 || T > kMaxTokens) ? MOE_ERR_SHAPE : MOE_OK; }

moe_status need(const void *p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    return aligned16(p) ? MOE_OK : MOE_ERR_ALIGN;
}
moe_status need_opt(const void *p) { return (p && !aligned16(p)) ? MOE_ERR_ALIGN : MOE_OK; }
moe_status need4(const void *p) {  // int32/fp32 vectors: 4-byte alignment
    if (!p) return MOE_ERR_INVALID_ARG;
    return ((uintptr_t)p & 3u) ? MOE_ERR_ALIGN : MOE_OK;
}
moe_status need4_opt(const void *p) { return (p && ((uintptr_t)p & 3u)) ? MOE_ERR_ALIGN : MOE_OK; }

#define TRY(x)                                      \
    do {                                            \
        moe_status _st = (x);                       \
        if (_st != MOE_OK) return _st;              \
    } while (0)
#define LAUNCH(x)                                   \
    do {                                            \
        if ((x) != hipSuccess) return MOE_ERR_LAUNCH; \
    } while (0)

// A current device, with the tiled kernels set up on it (once per device:
// every later call, also under graph capture, only reads that state).
moe_status device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_NO_DEVICE;
    if (tiled_gemm_prepare() != hipSuccess) return MOE_ERR_LAUNCH;
    return MOE_OK;
}

// Workspace carving for moe_layer_forward (every piece 256-byte aligned).
struct Layout {
    size_t logits, topk_idx, topk_w, shared_gate, counts, offsets, perm_src, inv_pos;
    size_t x_perm, x_scale, hm, y, shared_y, disp, tickets, total;
};

// Feature tiles of the tiled down projection: one combine ticket each.
constexpr int kCombTile = 256;
inline int comb_tiles(const moe_shape &s) { return (s.hidden + kCombTile - 1) / kCombTile; }

Layout layout(const moe_shape &s, int T) {
    Layout L;
    const size_t TK = (size_t)T * s.top_k;
    const size_t isz = act_bytes(s);
    const size_t xsz = s.dispatch == MOE_FP8_E4M3 ? 1 : isz;
    const size_t nsh = has_gate(s) ? (size_t)s.n_shared : 0;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o += up256(bytes);
        return at;
    };
    L.logits = take(route_ws_bytes(s, T));
    L.topk_idx = take(TK * 4);
    L.topk_w = take(TK * 4);
    L.shared_gate = take((size_t)T * 4);
    L.counts = take((size_t)s.n_slots * 4);
    L.offsets = take((size_t)(s.n_slots + 1) * 4);
    L.perm_src = take(TK * 4);
    L.inv_pos = take(TK * 4);
    L.x_perm = take(s.dispatch == MOE_FP8_E4M3 ? TK * s.hidden * xsz : 0);  // fp8 copies only
    L.x_scale = take(TK * 4);
    // routed rows [0, T*K), then the shared experts' rows (n_shared x T)
    L.hm = take((TK + nsh * T) * s.inter * isz);
    L.y = take((TK + nsh * T) * s.hidden * isz);
    L.shared_y = 0;  // inside y, after the routed rows
    L.disp = take(dispatch_scratch_bytes(T, s.top_k, s.n_slots));
    L.tickets = take((size_t)T * comb_tiles(s) * 4);  // fused combine (tiled down projection)
    L.total = o;
    return L;
}

template <typename P>
inline P at(void *ws, size_t off) {
    return reinterpret_cast<P>(reinterpret_cast<char *>(ws) + off);
}

// Groups expected to hold at least this many rows run on the LDS-tiled
// kernel (weight tiles reused across rows); fewer rows stream the weights.
constexpr int kTiledMinRows = 64;

bool use_tiled(long est_rows, int K, int dtype, int x_dtype) {
    return est_rows >= kTiledMinRows && tiled_gemm_supported_shape(K, dtype, x_dtype);
}

hipError_t gemm(const StreamArgs &a, int dtype, int x_dtype, int mode, int n_groups, int zblocks,
                long est_rows, long cap_rows, hipStream_t st) {
    if (a.n_sec == 0 && est_rows >= kTiledMinRows && tiled_gemm_supported(a, dtype, x_dtype))
        return launch_tiled_gemm(a, mode, n_groups, cap_rows / 128 + n_groups, st);
    if (a.comb.out) return hipErrorInvalidValue;  // the fused combine is the tiled kernel's
    return launch_stream_gemm(a, dtype, x_dtype, mode, n_groups, zblocks, est_rows, st);
}

int ffn_zblocks(int cap_rows, int n_groups) {
    if (n_groups <= 0) return 1;
    long per = ((long)cap_rows + n_groups - 1) / n_groups;
    long z = (per + 63) / 64;
    if (z < 1) z = 1;
    if (z > 16) z = 16;
    return (int)z;
}

// ------------------------------------------------------------ stage impls

hipError_t route_impl(const moe_shape &s, int T, const void *h, const void *w_router,
                      const float *bias, int32_t *topk_idx, float *topk_w, float *shared_gate,
                      float *logits_user, float *logits_buf, hipStream_t st) {
    const int gate = has_gate(s);
    const int N = s.n_experts + gate;
    StreamArgs a{};
    a.x = h;
    a.x_broadcast = 0;
    a.offsets = nullptr;
    a.rows_per_group = T;
    a.w0 = w_router;
    a.w1 = nullptr;
    a.w_group_stride = 0;
    a.out = logits_buf;
    a.out_ld = N;
    a.N = N;
    a.K = s.hidden;
    const RouterPlan plan = router_plan(s, T);
    a.ksplit = plan.ksplit;
    a.split_stride = (size_t)T * N;
    hipError_t e;
    if (plan.tiled) {
        e = launch_tiled_gemm(a, STREAM_LOGITS, 1, (T + 127) / 128, st);
    } else {
        const int rb = (T + 63) / 64;
        const int zb = rb * a.ksplit <= 65535 ? rb : 65535 / a.ksplit;  // rows stride by gridDim.z
        e = launch_stream_gemm(a, s.act, s.act, STREAM_LOGITS, 1, zb, T, st);
    }
    if (e != hipSuccess) return e;
    return launch_topk(logits_buf, a.ksplit, a.split_stride, N, T, s.n_experts, s.top_k, gate,
                       s.n_groups, s.topk_groups,
                       bias, topk_idx, topk_w, shared_gate, logits_user, st);
}

hipError_t dispatch_impl(const moe_shape &s, int T, const void *h, const int32_t *topk_idx,
                         const moe_slot_map &m, void *x_perm, float *x_scale, int32_t *counts,
                         int32_t *offsets, int32_t *perm_src, int32_t *inv_pos, void *scratch,
                         hipStream_t st, int32_t *tickets = nullptr) {
    DispatchArgs d{};
    d.T = T;
    d.K = s.top_k;
    d.E = s.n_experts;
    d.S = s.n_slots;
    d.H = s.hidden;
    d.dtype = s.act;
    d.x_dtype = s.dispatch;
    d.h = h;
    d.topk_idx = topk_idx;
    d.rep_off = m.rep_off;
    d.rep_slot = m.rep_slot;
    d.seed = m.seed;
    d.x_perm = x_perm;
    d.x_scale = x_scale;
    d.counts = counts;
    d.offsets = offsets;
    d.perm_src = perm_src;
    d.inv_pos = inv_pos;
    d.pair_code = reinterpret_cast<int32_t *>(scratch);
    d.chunk_counts = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(scratch) +
                                                 up256((size_t)T * s.top_k * 4));
    d.tickets = tickets;
    d.n_tiles = comb_tiles(s);
    return launch_dispatch(d, st);
}

// Secondary uniform groups riding in the same launch (shared experts).
struct Secondary {
    int n = 0;
    const void *x = nullptr;
    int x_broadcast = 0;
    const void *w0 = nullptr, *w1 = nullptr;
    int rows = 0, row_base = 0;
};

void set_secondary(StreamArgs &a, const Secondary &sec) {
    a.n_sec = sec.n;
    a.x2 = sec.x;
    a.x2_broadcast = sec.x_broadcast;
    a.w0b = sec.w0;
    a.w1b = sec.w1;
    a.rows2 = sec.rows;
    a.row2_base = sec.row_base;
}

hipError_t ffn_up_impl(const moe_shape &s, int n_groups, int zblocks, long est_rows,
                       long cap_rows, const void *x, int x_dtype, const float *x_scale,
                       int x_rows, const int32_t *gather, const int32_t *offsets,
                       int rows_per_group, const void *w_gate, const void *w_up, void *hm,
                       hipStream_t st, const Secondary &sec = Secondary()) {
    StreamArgs a{};
    set_secondary(a, sec);
    a.x = x;
    a.x_scale = x_scale;
    a.x_broadcast = x_rows == MOE_X_SHARED;
    a.gather = x_rows == MOE_X_GATHER ? gather : nullptr;
    a.gather_div = s.top_k;
    a.offsets = offsets;
    a.rows_per_group = rows_per_group;
    a.w0 = w_gate;
    a.w1 = w_up;
    a.w_group_stride = (size_t)s.inter * s.hidden;
    a.w_frag = s.w_layout == MOE_W_FRAG;
    a.out = hm;
    a.out_ld = s.inter;
    a.N = s.inter;
    a.K = s.hidden;
    a.ksplit = 1;
    return gemm(a, s.act, x_dtype, STREAM_SWIGLU, n_groups, zblocks, est_rows, cap_rows, st);
}

hipError_t ffn_down_impl(const moe_shape &s, int n_groups, int zblocks, long est_rows,
                         long cap_rows, const void *hm, const int32_t *offsets,
                         int rows_per_group, const void *w_down, void *y, hipStream_t st,
                         const Secondary &sec = Secondary(), const CombineArgs *comb = nullptr) {
    StreamArgs a{};
    set_secondary(a, sec);
    if (comb) a.comb = *comb;
    a.x = hm;
    a.offsets = offsets;
    a.rows_per_group = rows_per_group;
    a.w0 = w_down;
    a.w_group_stride = (size_t)s.hidden * s.inter;
    a.w_frag = s.w_layout == MOE_W_FRAG;
    a.out = y;
    a.out_ld = s.hidden;
    a.N = s.hidden;
    a.K = s.inter;
    a.ksplit = 1;
    return gemm(a, s.act, s.act, STREAM_STORE, n_groups, zblocks, est_rows, cap_rows, st);
}

CombineArgs combine_args(const moe_shape &s, int T, const void *y, const int32_t *inv_pos,
                         const float *topk_w, const void *shared_y, const float *shared_gate,
                         void *out) {
    CombineArgs c{};
    c.T = T;
    c.K = s.top_k;
    c.H = s.hidden;
    c.n_shared = shared_y ? s.n_shared : 0;
    c.dtype = s.act;
    c.y = y;
    c.inv_pos = inv_pos;
    c.topk_w = topk_w;
    c.shared_y = shared_y;
    c.shared_gate = shared_gate;
    c.out = out;
    return c;
}

hipError_t combine_impl(const moe_shape &s, int T, const void *y, const int32_t *inv_pos,
                        const float *topk_w, const void *shared_y, const float *shared_gate,
                        void *out, hipStream_t st) {
    return launch_combine(combine_args(s, T, y, inv_pos, topk_w, shared_y, shared_gate, out), st);
}

// Rows a group is expected to hold, used only to pick the kernel: cap_rows
// is T*K for the routed groups, spread about evenly over the E experts, and
// n_shared*T for the shared experts; cap/E keeps both choices alike for the
// staged and the fused entry points (outputs do not depend on the choice).
long est_group_rows(const moe_shape &s, long cap_rows) { return cap_rows / s.n_experts; }

moe_status check_ffn_common(const moe_shape *shape, int32_t n_groups, int32_t cap_rows) {
    TRY(check_shape(shape));
    if (n_groups < 1 || n_groups > 65535) return MOE_ERR_SHAPE;
    if (cap_rows < 0 || (int64_t)cap_rows > kMaxTokens * kMaxTopK) return MOE_ERR_SHAPE;
    return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------- ABI

MOE_EXPORT const char *moe_status_str(moe_status st) {
    switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_NO_DEVICE: return "MOE_ERR_NO_DEVICE";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
    case MOE_ERR_NOT_IMPLEMENTED: return "MOE_ERR_NOT_IMPLEMENTED";
    }
    return "MOE_ERR_UNKNOWN";
}

MOE_EXPORT const char *moe_version(void) { return "0.1.0"; }

MOE_EXPORT size_t moe_workspace_bytes(const moe_shape *shape, int32_t T) {
    if (check_shape(shape) != MOE_OK || check_T(T) != MOE_OK) return 0;
    return layout(*shape, T).total;
}

MOE_EXPORT moe_status moe_route(const moe_shape *shape, int32_t T, const void *h,
                                const void *w_router, const float *bias, int32_t *topk_idx,
                                float *topk_w, float *shared_gate, float *logits, void *ws,
                                size_t ws_bytes, void *stream) {
    TRY(check_shape(shape));
    TRY(check_T(T));
    if (T == 0) return MOE_OK;  // no token: nothing to route
    TRY(need(h));
    TRY(need(w_router));
    TRY(need4_opt(bias));
    TRY(need4(topk_idx));
    TRY(need4(topk_w));
    TRY(need4_opt(shared_gate));
    TRY(need4_opt(logits));
    if (has_gate(*shape) && !shared_gate) return MOE_ERR_INVALID_ARG;
    const size_t req = route_ws_bytes(*shape, T);
    if (!ws || ws_bytes < req) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    TRY(device_ok());
    LAUNCH(route_impl(*shape, T, h, w_router, bias, topk_idx, topk_w, shared_gate, logits,
                      reinterpret_cast<float *>(ws), (hipStream_t)stream));
    return MOE_OK;
}

MOE_EXPORT moe_status moe_dispatch(const moe_shape *shape, int32_t T, const void *h,
                                   const int32_t *topk_idx, const moe_slot_map *map,
                                   void *x_perm, float *x_scale, int32_t *counts,
                                   int32_t *offsets, int32_t *perm_src, int32_t *inv_pos,
                                   void *ws, size_t ws_bytes, void *stream) {
    TRY(check_shape(shape));
    TRY(check_T(T));
    if (!map) return MOE_ERR_INVALID_ARG;
    TRY(need4(counts));
    TRY(need4(offsets));
    if (T > 0) {  // with no token only counts and offsets are written
        TRY(need(h));
        TRY(need4(topk_idx));
        TRY(need4(map->rep_off));
        TRY(need4(map->rep_slot));
        if (shape->dispatch == MOE_FP8_E4M3) {  // quantised rows must be stored
            TRY(need(x_perm));
            TRY(need4(x_scale));
        } else {
            TRY(need_opt(x_perm));  // NULL: indices only, the GEMM gathers rows
        }
        TRY(need4(perm_src));
        TRY(need4(inv_pos));
    }
    const size_t req = dispatch_scratch_bytes(T, shape->top_k, shape->n_slots);
    if (!ws || ws_bytes < req) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    TRY(device_ok());
    LAUNCH(dispatch_impl(*shape, T, h, topk_idx, *map, x_perm, x_scale, counts, offsets,
                         perm_src, inv_pos, ws, (hipStream_t)stream));
    return MOE_OK;
}

MOE_EXPORT moe_status moe_expert_ffn_up(const moe_shape *shape, int32_t n_groups,
                                        int32_t cap_rows, const void *x, int32_t x_dtype,
                                        const float *x_scale, int32_t x_rows,
                                        const int32_t *gather, const int32_t *offsets,
                                        const void *w_gate, const void *w_up, void *hm,
                                        void *stream) {
    TRY(check_ffn_common(shape, n_groups, cap_rows));
    if (x_dtype != shape->act && !(x_dtype == MOE_FP8_E4M3 && shape->act == MOE_F16))
        return MOE_ERR_DTYPE;
    if (x_rows != MOE_X_PERMUTED && x_rows != MOE_X_SHARED && x_rows != MOE_X_GATHER)
        return MOE_ERR_INVALID_ARG;
    if (x_rows == MOE_X_GATHER) {
        TRY(need4(gather));
        if (x_dtype == MOE_FP8_E4M3) return MOE_ERR_DTYPE;  // fp8 rows are dispatched copies
    }
    TRY(need(x));
    if (x_dtype == MOE_FP8_E4M3) TRY(need4(x_scale));
    TRY(need4(offsets));
    TRY(need(w_gate));
    TRY(need(w_up));
    TRY(need(hm));
    if (cap_rows == 0) return MOE_OK;
    TRY(device_ok());
    LAUNCH(ffn_up_impl(*shape, n_groups, ffn_zblocks(cap_rows, n_groups),
                       est_group_rows(*shape, cap_rows), cap_rows, x, x_dtype, x_scale, x_rows,
                       gather, offsets, 0, w_gate, w_up, hm, (hipStream_t)stream));
    return MOE_OK;
}

MOE_EXPORT moe_status moe_expert_ffn_down(const moe_shape *shape, int32_t n_groups,
                                          int32_t cap_rows, const void *hm,
                                          const int32_t *offsets, const void *w_down, void *y,
                                          void *stream) {
    TRY(check_ffn_common(shape, n_groups, cap_rows));
    TRY(need(hm));
    TRY(need4(offsets));
    TRY(need(w_down));
    TRY(need(y));
    if (cap_rows == 0) return MOE_OK;
    TRY(device_ok());
    LAUNCH(ffn_down_impl(*shape, n_groups, ffn_zblocks(cap_rows, n_groups),
                         est_group_rows(*shape, cap_rows),
                         cap_rows, hm, offsets, 0, w_down, y, (hipStream_t)stream));
    return MOE_OK;
}

MOE_EXPORT moe_status moe_expert_ffn(const moe_shape *shape, int32_t n_groups, int32_t cap_rows,
                                     const void *x, int32_t x_dtype, const float *x_scale,
                                     int32_t x_rows, const int32_t *gather,
                                     const int32_t *offsets, const void *w_gate,
                                     const void *w_up, const void *w_down, void *y, void *ws,
                                     size_t ws_bytes, void *stream) {
    TRY(check_ffn_common(shape, n_groups, cap_rows));
    const size_t req = up256((size_t)cap_rows * shape->inter * act_bytes(*shape));
    if (cap_rows > 0 && (!ws || ws_bytes < req)) return MOE_ERR_WORKSPACE;
    if (cap_rows > 0 && !aligned16(ws)) return MOE_ERR_ALIGN;
    TRY(need(w_down));
    TRY(need(y));
    moe_status st = moe_expert_ffn_up(shape, n_groups, cap_rows, x, x_dtype, x_scale, x_rows,
                                      gather, offsets, w_gate, w_up, ws, stream);
    if (st != MOE_OK) return st;
    return moe_expert_ffn_down(shape, n_groups, cap_rows, ws, offsets, w_down, y, stream);
}

MOE_EXPORT moe_status moe_combine(const moe_shape *shape, int32_t T, const void *y,
                                  const int32_t *inv_pos, const float *topk_w,
                                  const void *shared_y, const float *shared_gate, void *out,
                                  void *stream) {
    TRY(check_shape(shape));
    TRY(check_T(T));
    if (T == 0) return MOE_OK;
    TRY(need(y));
    TRY(need4(inv_pos));
    TRY(need4(topk_w));
    TRY(need_opt(shared_y));
    if (shared_y) TRY(need4(shared_gate));
    TRY(need(out));
    TRY(device_ok());
    LAUNCH(combine_impl(*shape, T, y, inv_pos, topk_w, shared_y, shared_gate, out,
                        (hipStream_t)stream));
    return MOE_OK;
}

MOE_EXPORT moe_status moe_expert_counts(const moe_shape *shape, int32_t T,
                                        const int32_t *topk_idx, int32_t *counts, void *stream) {
    TRY(check_shape(shape));
    TRY(check_T(T));
    TRY(need4(counts));
    if (T > 0) TRY(need4(topk_idx));
    TRY(device_ok());
    LAUNCH(launch_expert_counts(topk_idx, (long)T * shape->top_k, shape->n_experts, counts,
                                (hipStream_t)stream));
    return MOE_OK;
}

MOE_EXPORT moe_status moe_pack_weights(int32_t dtype, int64_t n_mats, int32_t rows,
                                       int32_t cols, const void *src, void *dst, void *stream) {
    if (dtype != MOE_F16 && dtype != MOE_F32) return MOE_ERR_DTYPE;
    const int esize = dtype == MOE_F16 ? 2 : 4;
    if (n_mats < 0 || n_mats > kMaxPackMats) return MOE_ERR_SHAPE;
    if (rows < 16 || rows > kMaxDim || rows % 16) return MOE_ERR_SHAPE;
    if (cols < 1 || cols > kMaxDim || ((int64_t)cols * esize) % 64) return MOE_ERR_SHAPE;
    TRY(need(src));
    TRY(need(dst));
    const uint64_t bytes = (uint64_t)n_mats * (uint64_t)rows * (uint64_t)cols * (uint64_t)esize;
    const uint64_t a = (uint64_t)(uintptr_t)src, b = (uint64_t)(uintptr_t)dst;
    if (bytes > 0 && a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlap
    if (n_mats == 0) return MOE_OK;
    TRY(device_ok());
    LAUNCH(launch_pack_frag(src, dst, (long)n_mats, rows, cols * esize, (hipStream_t)stream));
    return MOE_OK;
}

MOE_EXPORT moe_status moe_layer_forward(const moe_shape *shape, const moe_weights *w,
                                        const moe_slot_map *map, int32_t T, const void *h,
                                        void *out, void *ws, size_t ws_bytes, void *stream) {
    return moe::layer_forward_run(shape, w, map, T, h, out, ws, ws_bytes, nullptr, stream);
}

MOE_EXPORT moe_status moe_layer_forward_profiled(const moe_shape *shape, const moe_weights *w,
                                                 const moe_slot_map *map, int32_t T,
                                                 const void *h, void *out, void *ws,
                                                 size_t ws_bytes, const moe_profile *prof,
                                                 void *stream) {
    if (!prof) return MOE_ERR_INVALID_ARG;
    return moe::layer_forward_run(shape, w, map, T, h, out, ws, ws_bytes, prof, stream);
}

namespace moe {

moe_status layer_forward_validate(const moe_shape *shape, const moe_weights *w,
                                  const moe_slot_map *map, int32_t T, const void *h, void *out) {
    TRY(check_shape(shape));
    TRY(check_T(T));
    if (!w || !map) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;  // no token: nothing else is read
    TRY(need(h));
    TRY(need(out));
    TRY(need(w->w_router));
    TRY(need4_opt(w->bias));
    TRY(need(w->w_gate));
    TRY(need(w->w_up));
    TRY(need(w->w_down));
    TRY(need4(map->rep_off));
    TRY(need4(map->rep_slot));
    if (has_gate(*shape)) {
        TRY(need(w->sh_gate));
        TRY(need(w->sh_up));
        TRY(need(w->sh_down));
    }
    return MOE_OK;
}

moe_status layer_forward_run(const moe_shape *shape, const moe_weights *w,
                             const moe_slot_map *map, int32_t T, const void *h, void *out,
                             void *ws, size_t ws_bytes, const moe_profile *prof, void *stream) {
    TRY(layer_forward_validate(shape, w, map, T, h, out));
    if (T == 0) return MOE_OK;  // no token: empty output
    const moe_shape &s = *shape;
    const int gate = has_gate(s);
    const Layout L = layout(s, T);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    TRY(device_ok());
    hipStream_t st = (hipStream_t)stream;
    auto mark = [&](int i) -> bool {
        return !prof || !prof->events[i] ||
               hipEventRecord((hipEvent_t)prof->events[i], st) == hipSuccess;
    };
#define MARK(i)                                  \
    do {                                         \
        if (!mark(i)) return MOE_ERR_LAUNCH;     \
    } while (0)

    int32_t *topk_idx = at<int32_t *>(ws, L.topk_idx);
    float *topk_w = at<float *>(ws, L.topk_w);
    float *sgate = at<float *>(ws, L.shared_gate);
    int32_t *offsets = at<int32_t *>(ws, L.offsets);
    int32_t *inv_pos = at<int32_t *>(ws, L.inv_pos);
    float *x_scale = at<float *>(ws, L.x_scale);
    const int cap = T * s.top_k;

    MARK(0);
    LAUNCH(route_impl(s, T, h, w->w_router, w->bias, topk_idx, topk_w, gate ? sgate : nullptr,
                      nullptr, at<float *>(ws, L.logits), st));
    MARK(1);
    // fp8 rows are quantised copies; otherwise the gate/up GEMM gathers the
    // hidden rows through perm_src and dispatch writes indices only
    const bool copy_rows = s.dispatch == MOE_FP8_E4M3;
    int32_t *perm_src = at<int32_t *>(ws, L.perm_src);
    const int z = ffn_zblocks(cap, s.n_slots);
    const long est = est_group_rows(s, cap);
    // MOE_F_FUSED_COMBINE, where the routed down projection runs on the
    // LDS-tiled kernel: the combine rides in its tail (tickets seeded by
    // dispatch).  Otherwise the separate combine launch.
    const bool fuse = (s.flags & MOE_F_FUSED_COMBINE) && use_tiled(est, s.inter, s.act, s.act);
    int32_t *tickets = fuse ? at<int32_t *>(ws, L.tickets) : nullptr;
    LAUNCH(dispatch_impl(s, T, h, topk_idx, *map, copy_rows ? at<void *>(ws, L.x_perm) : nullptr,
                         x_scale, at<int32_t *>(ws, L.counts), offsets, perm_src, inv_pos,
                         at<void *>(ws, L.disp), st, tickets));
    MARK(2);
    void *hm = at<void *>(ws, L.hm), *y = at<void *>(ws, L.y);
    const size_t isz = act_bytes(s);
    void *shared_y = gate ? (void *)((char *)y + (size_t)cap * s.hidden * isz) : nullptr;
    const void *x_routed = copy_rows ? at<void *>(ws, L.x_perm) : h;
    const int x_mode = copy_rows ? MOE_X_PERMUTED : MOE_X_GATHER;
    const long cap_sh = (long)s.n_shared * T;
    const long est_sh = est_group_rows(s, cap_sh);
    // The shared experts (every token, Step 5) ride in the routed launches as
    // secondary groups when both stream their weights with the kernels the
    // separate calls would pick for each (so the sums, and the output, are
    // bitwise those of the staged calls); rows cap.. of hm/y.
    const bool merged = gate && !copy_rows && !fuse && !use_tiled(est, s.hidden, s.act, s.act) &&
                        !use_tiled(est_sh, s.hidden, s.act, s.act) &&
                        stream_gemm_same_kernel(s.act, STREAM_STORE, est, est_sh);
    if (merged) {
        Secondary up_sec, down_sec;
        up_sec.n = down_sec.n = s.n_shared;
        up_sec.x = h;
        up_sec.x_broadcast = 1;
        up_sec.w0 = w->sh_gate;
        up_sec.w1 = w->sh_up;
        down_sec.x = hm;
        down_sec.w0 = w->sh_down;
        up_sec.rows = down_sec.rows = T;
        up_sec.row_base = down_sec.row_base = cap;
        LAUNCH(ffn_up_impl(s, s.n_slots, z, est, cap, x_routed, s.dispatch, x_scale, x_mode,
                           perm_src, offsets, 0, w->w_gate, w->w_up, hm, st, up_sec));
        MARK(3);
        LAUNCH(ffn_down_impl(s, s.n_slots, z, est, cap, hm, offsets, 0, w->w_down, y, st,
                             down_sec));
    } else {
        LAUNCH(ffn_up_impl(s, s.n_slots, z, est, cap, x_routed, s.dispatch, x_scale, x_mode,
                           perm_src, offsets, 0, w->w_gate, w->w_up, hm, st));
        MARK(3);
        auto shared_ffn = [&]() -> hipError_t {
            const int zs = (T + 63) / 64 < 65535 ? (T + 63) / 64 : 65535;
            void *hm_sh = (char *)hm + (size_t)cap * s.inter * isz;
            hipError_t e = ffn_up_impl(s, s.n_shared, zs, est_sh, cap_sh, h, s.act, nullptr,
                                       MOE_X_SHARED, nullptr, nullptr, T, w->sh_gate, w->sh_up,
                                       hm_sh, st);
            if (e != hipSuccess) return e;
            return ffn_down_impl(s, s.n_shared, zs, est_sh, cap_sh, hm_sh, nullptr, T, w->sh_down,
                                 shared_y, st);
        };
        if (fuse) {
            // the shared rows first: the routed launch's tail reads them
            if (gate) LAUNCH(shared_ffn());
            CombineArgs c = combine_args(s, T, y, inv_pos, topk_w, shared_y, sgate, out);
            c.perm_src = perm_src;
            c.tickets = tickets;
            LAUNCH(ffn_down_impl(s, s.n_slots, z, est, cap, hm, offsets, 0, w->w_down, y, st,
                                 Secondary(), &c));
        } else {
            LAUNCH(ffn_down_impl(s, s.n_slots, z, est, cap, hm, offsets, 0, w->w_down, y, st));
            if (gate) LAUNCH(shared_ffn());
        }
    }
    MARK(4);
    if (!fuse)
        LAUNCH(combine_impl(s, T, at<void *>(ws, L.y), inv_pos, topk_w, shared_y, sgate, out, st));
    MARK(5);
#undef MARK
    return MOE_OK;
}
}  // namespace moe
