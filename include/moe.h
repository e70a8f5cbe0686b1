/*
 * moe.h -- C ABI of libmoe: one DeepSeek-V3-style MoE layer on one MI355X.
 *
 * The operations follow the five-step token journey of the expert-parallelism
 * blog page (yveltals, "专家并行（EP）", section 2.2):
 *   Step 1  router linear + top-K            -> moe_route
 *   Step 2  dispatch to the experts' owners  -> moe_dispatch (an on-device
 *           permutation into per-slot contiguous groups: one GPU holds this
 *           rank's share of the experts, so nothing crosses a link)
 *   Step 3  expert FFN                       -> moe_expert_ffn
 *                                               (= moe_expert_ffn_up + _down)
 *   Step 4  combine (return the outputs)     -> moe_combine
 *   Step 5  gate-weighted sum + shared term     (same call)
 *   all of it                                -> moe_layer_forward
 *
 * Conventions for every call
 *   - Pointers are DEVICE memory unless marked (host).  The caller allocates
 *     and owns every buffer; the library never allocates, frees or
 *     synchronises.  State it keeps across calls, per device: the number of
 *     resident workgroups of each LDS-tiled GEMM kernel (counted for every
 *     such kernel at once, after raising its dynamic LDS limit with
 *     hipFuncSetAttribute, on the first call of any entry point on the
 *     device; later calls read it), and the device address of
 *     moe_layer_forward_noalloc's static workspace array (looked up on that
 *     entry point's first call on the device).  Both are set up race-free;
 *     every entry point may be called from several host threads.
 *   - Matrices are row-major and "out-major": a weight that maps an input of
 *     length n to m outputs is stored [m][n], i.e. the transpose of the
 *     page's [in, out] math shapes (router [7168, 256], gate/up
 *     [7168, 2048], down [2048, 7168]).  Every row starts 16-byte aligned.
 *     Expert weights (routed and shared) may instead be in the fragment
 *     layout MOE_W_FRAG (moe_shape.w_layout, moe_pack_weights).
 *   - dtype: MOE_F16 (fp16 activations and weights, fp32 accumulation,
 *     fp16 outputs) or MOE_F32 (fp32 throughout).  Dispatched rows may be
 *     MOE_FP8_E4M3 with one fp32 scale per row (F16 layers only).
 *   - stream: a hipStream_t; NULL is the default stream.  Every call only
 *     enqueues work on it and returns; outputs are valid once the stream
 *     reaches that point.  The work is kernel launches only (no copy,
 *     memset, allocation or synchronisation), so calls may be captured
 *     into a HIP graph and replayed, after one eager call per device that
 *     sets up the per-device state above (any entry point; for
 *     moe_layer_forward_noalloc, that entry point itself).
 *   - Return value: a synchronous status from host-side validation (shapes,
 *     NULL pointers, alignment, dtype combinations, workspace size), or
 *     MOE_ERR_LAUNCH if a kernel launch was rejected.  Nothing is enqueued
 *     when validation fails.  Faults inside kernels surface at the caller's
 *     next synchronisation of the stream.  No C++ exception crosses the ABI.
 *   - Limits: hidden and inter positive multiples of 128, at most 65536;
 *     1 <= top_k <= min(E, 16); E <= 1024; 1 <= S <= 1024; n_shared <= 16;
 *     0 <= T <= 2^20 (T = 0 is valid: no token, nothing routed).
 *   - Routing preconditions: a token's top_k experts are distinct (the
 *     router never repeats one) and each local slot is listed under one
 *     expert (a slot holds one expert's weights).  Dispatch keeps its
 *     output well defined when they are broken: of two pairs of one token
 *     that would meet in one slot, only the earlier k is dispatched (the
 *     later gets inv_pos = -1 and contributes nothing).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,     /* NULL pointer / bad flag */
    MOE_ERR_SHAPE = 2,           /* dims outside the limits above */
    MOE_ERR_DTYPE = 3,           /* unsupported dtype combination */
    MOE_ERR_ALIGN = 4,           /* pointer not 16-byte aligned */
    MOE_ERR_WORKSPACE = 5,       /* ws NULL or ws_bytes too small */
    MOE_ERR_NO_DEVICE = 6,       /* no HIP device usable */
    MOE_ERR_LAUNCH = 7,          /* a kernel launch failed */
    MOE_ERR_NOT_IMPLEMENTED = 8
} moe_status;

typedef enum { MOE_F32 = 0, MOE_F16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* moe_shape.flags */
#define MOE_F_SHARED 1u /* layer has shared experts: add their gated sum */
/* moe_layer_forward only, where the routed down projection runs on the
 * LDS-tiled kernel (fp16, >= 64 expected rows per slot: prefill batches):
 * form the output in that launch's tail instead of a separate combine
 * launch (EP blog section 2.3: the combine may run alongside the last
 * expert computations; large-EP article 三.2: fused gather-GEMM-scatter).
 * Dispatch seeds one ticket per (token, 256-feature tile) with the token's
 * local pair count; the workgroup that writes the last of a tile's rows
 * (agent-scope release, atomic decrement, acquire) sums the token's rows in
 * k order with the combine's arithmetic, so the output is bitwise the same.
 * Off by default: on MI355X at 16,384 tokens (EP=8 share) the layer takes
 * about 2.0 ms with it against 1.7 ms with the separate combine -- the sums
 * of the last-completed tiles fall on the workgroups that finish last, while
 * the matrix cores idle.  Ignored by the staged entry points. */
#define MOE_F_FUSED_COMBINE 2u

/* moe_shape.w_layout: how the expert weights (w_gate, w_up, w_down and the
 * shared experts' sh_*) of a layer are stored; the router stays row-major.
 *   MOE_W_ROWMAJOR  each matrix [rows][cols] row-major.
 *   MOE_W_FRAG      each matrix [rows][cols] (rows % 16 == 0, a row of
 *                   rb = cols * esize bytes, rb % 64 == 0) as 1 KB fragments:
 *                   fragment (i, j), i < rows / 16, j < rb / 64, sits at byte
 *                   (i * (rb / 64) + j) * 1024 of the matrix and holds rows
 *                   16i .. 16i+15 x row bytes 64j .. 64j+63; its byte
 *                   256 q + 16 r + c (q < 4, r < 16, c < 16) is byte
 *                   64j + 16q + c of row 16i + r.  That is the operand layout
 *                   of the matrix cores' 16 x 16 x 32 fp16 product, one
 *                   16-byte piece per lane, so the expert GEMMs read each
 *                   operand tile as one contiguous 1 KB (decode streams the
 *                   weights about 11% faster on MI355X).  A matrix keeps its
 *                   size and position: slot s of w_gate still starts at
 *                   element s * I * H.  moe_pack_weights converts. */
#define MOE_W_ROWMAJOR 0
#define MOE_W_FRAG 1

/* Where the expert GEMM finds the input row of output row r of group g
 * (x_rows argument of moe_expert_ffn_up / moe_expert_ffn). */
#define MOE_X_PERMUTED 0 /* x[r]: rows already permuted (moe_dispatch's x_perm) */
#define MOE_X_SHARED 1   /* x[r - offsets[g]]: every group reads the same rows */
#define MOE_X_GATHER 2   /* x[gather[r] / top_k]: gather = perm_src from
                            moe_dispatch, x = h (fp16/fp32 rows only) */

/* Layer description (host struct). */
typedef struct {
    int32_t hidden;    /* H: 7168 for DeepSeek-V3 (section 2.2, Step 1) */
    int32_t inter;     /* I: 2048 (section 一: gate/up [7168, 2048]) */
    int32_t n_experts; /* E: routed experts the router scores (256) */
    int32_t top_k;     /* K: experts per token (8) */
    int32_t n_slots;   /* S: expert weight sets resident here (32 for one
                          rank of EP=8, 33 with a redundant replica, 256 for
                          the whole layer; sections 2.1 and 6.3) */
    int32_t n_shared;  /* shared experts (2 in DeepSeek-V3, section 2.1) */
    int32_t act;       /* moe_dtype of h, weights and outputs: F32 or F16 */
    int32_t dispatch;  /* moe_dtype of dispatched rows: == act, or FP8_E4M3 */
    uint32_t flags;    /* MOE_F_SHARED, MOE_F_FUSED_COMBINE */
    /* Group-limited routing (the outlook of section 八: route to expert
     * groups first, then to experts).  n_groups = 0: off.  Otherwise the E
     * experts form n_groups contiguous groups of E / n_groups (a group is
     * one EP rank's range, section 2.1); a group's score is its largest
     * logit; only the topk_groups best groups (ties: lower group id) are
     * eligible for the top-K.  Gates stay the softmax over all E logits.
     * Limits: n_groups divides E, n_groups <= 64,
     * 1 <= topk_groups <= n_groups, top_k <= topk_groups * E / n_groups. */
    int32_t n_groups;
    int32_t topk_groups;
    int32_t w_layout;  /* MOE_W_ROWMAJOR or MOE_W_FRAG (other values:
                          MOE_ERR_INVALID_ARG) */
} moe_shape;

/* Expert -> local slot table (device arrays), sections 2.1 and 6.3.
 * Expert e has n_e = rep_off[e+1] - rep_off[e] replicas, listed in
 * rep_slot[rep_off[e] .. rep_off[e+1]): a local slot in [0, S) or -1 for a
 * copy that lives on another GPU.  A pair (t, k) routed to e goes to replica
 * splitmix64(seed ^ (t*K + k)) mod n_e (SplitMix64 output function, Steele,
 * Lea and Flood 2014); n_e == 1 needs no hash; n_e == 0 means not here. */
typedef struct {
    const int32_t *rep_off;  /* [E + 1] */
    const int32_t *rep_slot; /* [rep_off[E]] */
    uint64_t seed;
} moe_slot_map;

/* Weights of the whole layer (device pointers; dtype = shape.act). */
typedef struct {
    const void *w_router; /* [E][H]; with MOE_F_SHARED, [E + 1][H]: row E is
                             the shared-expert gate vector w_sg */
    const float *bias;    /* [E] fp32 router logit bias, or NULL */
    const void *w_gate;   /* [S][I][H] */
    const void *w_up;     /* [S][I][H] */
    const void *w_down;   /* [S][H][I] */
    const void *sh_gate;  /* [n_shared][I][H]  (MOE_F_SHARED only) */
    const void *sh_up;    /* [n_shared][I][H] */
    const void *sh_down;  /* [n_shared][H][I] */
} moe_weights;

/* Step 1 (section 2.2): router linear and top-K.
 *   logits[t][e] = fp32(sum_i h[t][i] * w_router[e][i]) + bias[e]
 *   p[t] = softmax over all E logits; the K experts with the largest logits
 *   (ties: lower id first; with shape.n_groups > 0 only experts of the
 *   topk_groups best groups) are written to topk_idx[t][0..K) in that order
 *   and their probabilities, not renormalised, to topk_w[t][0..K).
 *   With MOE_F_SHARED, shared_gate[t] = sigmoid(h[t] . w_router[E]).
 * h [T][H] (act); topk_idx int32 [T][K]; topk_w fp32 [T][K];
 * shared_gate fp32 [T] or NULL; logits fp32 [T][E] or NULL (if non-NULL the
 * raw logits including bias are stored).
 * Workspace: ws of moe_workspace_bytes(shape, T) bytes (holds the fp32
 * partial logits of the K-split router GEMM). */
moe_status moe_route(const moe_shape *shape, int32_t T, const void *h,
                     const void *w_router, const float *bias, int32_t *topk_idx,
                     float *topk_w, float *shared_gate, float *logits, void *ws,
                     size_t ws_bytes, void *stream);

/* Step 2 (section 2.2) on one GPU: permute the local (token, k) pairs into
 * per-slot contiguous groups.  slot(t, k) comes from `map`; rows are ordered
 * by (slot, t) ascending; no capacity limit, nothing dropped.
 *   counts [S]         rows per slot
 *   offsets [S + 1]    exclusive prefix sum; offsets[S] = local rows P
 *   perm_src [T*K]     perm_src[row] = t*K + k for row < P (rest untouched)
 *   inv_pos [T][K]     row of pair (t, k), or -1 if the pair is not local
 *   x_perm [T*K][H]    x_perm[row] = h[t]; with dispatch = FP8_E4M3 the row
 *                      is stored as OCP E4M3 codes (uint8) with
 *                      x_scale[row] = amax/448 and codes
 *                      E4M3_RNE(clamp(h * (448/amax), -448, 448)) (section
 *                      2.3: FP8 halves the dispatch payload); x_scale may be
 *                      NULL otherwise.  Rows >= P are untouched.  Without
 *                      FP8, x_perm may be NULL: only the indices are written
 *                      and the gate/up GEMM gathers h rows (MOE_X_GATHER).
 * Workspace: ws of at least moe_workspace_bytes(shape, T) bytes. */
moe_status moe_dispatch(const moe_shape *shape, int32_t T, const void *h,
                        const int32_t *topk_idx, const moe_slot_map *map, void *x_perm,
                        float *x_scale, int32_t *counts, int32_t *offsets,
                        int32_t *perm_src, int32_t *inv_pos, void *ws, size_t ws_bytes,
                        void *stream);

/* Step 3, first half (section 一 gives gate/up [7168, 2048]): for every group
 * g < n_groups and every row r in [offsets[g], offsets[g+1]):
 *   hm[r] = silu(w_gate[g] . x_r) * (w_up[g] . x_r),  silu(z) = z*sigmoid(z)
 * x_r per x_rows: MOE_X_PERMUTED x[r]; MOE_X_SHARED x[r - offsets[g]] (how
 * the shared experts see all tokens); MOE_X_GATHER x[gather[r] / top_k]
 * (gather int32 [cap_rows], NULL otherwise).  With x_dtype FP8_E4M3 (only
 * with MOE_X_PERMUTED) the row is decoded and multiplied by x_scale[r].
 * hm [cap_rows][I] (act).  cap_rows (host) bounds offsets[n_groups]; groups
 * with no rows read no weights. */
moe_status moe_expert_ffn_up(const moe_shape *shape, int32_t n_groups, int32_t cap_rows,
                             const void *x, int32_t x_dtype, const float *x_scale,
                             int32_t x_rows, const int32_t *gather, const int32_t *offsets,
                             const void *w_gate, const void *w_up, void *hm, void *stream);

/* Step 3, second half (section 6.3's 88 MB per expert = three 7168 x 2048
 * fp16 matrices, so down is [2048, 7168]):  y[r] = w_down[g] . hm[r].
 * y [cap_rows][H] (act). */
moe_status moe_expert_ffn_down(const moe_shape *shape, int32_t n_groups, int32_t cap_rows,
                               const void *hm, const int32_t *offsets, const void *w_down,
                               void *y, void *stream);

/* Step 3 whole: up then down, with hm in the workspace. */
moe_status moe_expert_ffn(const moe_shape *shape, int32_t n_groups, int32_t cap_rows,
                          const void *x, int32_t x_dtype, const float *x_scale,
                          int32_t x_rows, const int32_t *gather, const int32_t *offsets,
                          const void *w_gate, const void *w_up, const void *w_down, void *y,
                          void *ws, size_t ws_bytes, void *stream);

/* Steps 4 and 5 (section 2.2):
 *   out[t] = sum_{k = 0..K-1, inv_pos[t][k] >= 0} topk_w[t][k] * y[inv_pos[t][k]]
 *          + shared_gate[t] * sum_j shared_y[j][t]      (if shared_y != NULL)
 * summed in k order in fp32, rounded once to act.  A token with no local
 * pair and no shared term gets exact zeros (a rank's partial output).
 * y [*][H]; shared_y [n_shared][T][H] or NULL; out [T][H] (act). */
moe_status moe_combine(const moe_shape *shape, int32_t T, const void *y,
                       const int32_t *inv_pos, const float *topk_w, const void *shared_y,
                       const float *shared_gate, void *out, void *stream);

/* Expert weights into the fragment layout (see MOE_W_FRAG), once, when
 * they are loaded: dst[m] = MOE_W_FRAG form of the row-major src[m], for
 * n_mats matrices [rows][cols] of dtype MOE_F16 or MOE_F32 stored back to
 * back (e.g. all S slots of w_gate: n_mats = S, rows = I, cols = H).
 * Limits: 16 <= rows <= 65536, rows % 16 == 0; 1 <= cols <= 65536,
 * cols * esize % 64 == 0; 0 <= n_mats <= 2^20 (0: nothing enqueued).
 * src and dst are 16-byte aligned and must not overlap
 * (MOE_ERR_INVALID_ARG); the caller owns both.  A pure permutation: the
 * products over the packed weights are bitwise those over the row-major
 * ones. */
moe_status moe_pack_weights(int32_t dtype, int64_t n_mats, int32_t rows, int32_t cols,
                            const void *src, void *dst, void *stream);

/* Steps 1-5 for T tokens: moe_route, moe_dispatch, moe_expert_ffn on the
 * routed groups and (MOE_F_SHARED) on the shared experts, moe_combine.
 * Same kernels and order as the staged calls, so the outputs are bitwise
 * equal to the staged path (with MOE_F_FUSED_COMBINE the combine runs in
 * the down projection's tail instead, with the same arithmetic: still
 * bitwise equal).  out [T][H] (act).  Without MOE_F_SHARED the
 * output is this GPU's partial sum over its local pairs. */
moe_status moe_layer_forward(const moe_shape *shape, const moe_weights *weights,
                             const moe_slot_map *map, int32_t T, const void *h, void *out,
                             void *ws, size_t ws_bytes, void *stream);

/* Profiling variant of moe_layer_forward for benchmarks: the same kernels
 * in the same order, and additionally records the caller's events
 * (hipEvent_t created by the caller; NULL entries are skipped) on the
 * stream at the stage boundaries: events[0] before Step 1, [1] after the
 * router (Step 1), [2] after dispatch (Step 2), [3] after the gate/up GEMM,
 * [4] after the down GEMM and the shared experts, [5] after combine
 * (Steps 4-5).  An event record that fails returns MOE_ERR_LAUNCH. */
typedef struct {
    void *events[6];
} moe_profile;

moe_status moe_layer_forward_profiled(const moe_shape *shape, const moe_weights *weights,
                                      const moe_slot_map *map, int32_t T, const void *h,
                                      void *out, void *ws, size_t ws_bytes,
                                      const moe_profile *prof, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_layer_forward -- same kernels and order, so the output is
 * bitwise equal -- with the workspace held by the library: one static
 * device array of MOE_NOALLOC_SCRATCH_BYTES per device, kept until the
 * process ends and looked up on the first call on each device.  Nothing is
 * allocated or freed.  Shapes whose moe_workspace_bytes(shape, T) exceeds
 * the array return MOE_ERR_WORKSPACE with nothing enqueued (64 MiB holds
 * DeepSeek-V3 decode batches up to 256 tokens: 39.6 MiB for one EP=8
 * rank's 32 experts, 48.6 MiB for the whole layer with 2 shared experts).
 * Every call on one device uses the same array: calls that overlap on a
 * GPU (other streams, other threads) race and must be ordered by the
 * caller.  Other arguments and errors as moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_shape *shape, const moe_weights *weights,
                                     const moe_slot_map *map, int32_t T, const void *h,
                                     void *out, void *stream);

/* ------------------------------------------------------------------
 * EPLB-lite: the load balancer of section 6.2 with the redundant copies of
 * section 6.3, for one EP group of n_ranks GPUs (expert e's home is rank
 * e / (E / n_ranks), section 2.1).
 *   monitor  moe_expert_counts (device) gives one forward's per-expert
 *            token counts; moe_eplb_observe pushes them (host copy) into a
 *            sliding window of the last `window` forwards.  A rank's load is
 *            the sum over the copies it holds of count_e / n_copies_e (a
 *            token picks one of an expert's copies uniformly, section 6.3),
 *            accumulated in expert order in double precision.
 *   detect   max rank load / mean rank load > threshold (1.2 on the page).
 *   migrate  moe_eplb_rebalance: greedily, up to max_moves times, the copy
 *            with the largest per-copy load on the most loaded rank (ties:
 *            lower expert id; skipping experts that cannot be placed) gets a
 *            new copy on the least loaded rank (ties: lower rank) that holds
 *            none and has one of its spare_slots free.  Home copies stay.
 *   tables   moe_eplb_slot_map writes one rank's moe_slot_map arrays for
 *            the current placement: home experts in slots 0..E/R-1, spare
 *            slots after them; each expert lists its copies in the order
 *            they were created (the home copy first while it lives), a copy
 *            on another rank as -1.  The new expert weights must be in place
 *            before a forward uses the new table; keep the old table for
 *            work already queued (the page's double-buffered routing table).
 *   cleanup  moe_eplb_cleanup, called once all work queued with the old
 *            table has finished: the copy each migration since the last
 *            cleanup was taken from (its original position on the
 *            overloaded rank) is reclaimed, unless it is the expert's last
 *            copy -- the migration becomes a move (the page's optional
 *            step 4).  A reclaimed home slot stays empty; a reclaimed spare
 *            slot becomes a hole that the next copy placed on that rank
 *            fills, so slot numbers never shift.
 * The monitor state is caller memory of moe_eplb_state_bytes(cfg) bytes;
 * these calls are host-only and never touch a device.  Calls on one state
 * must not overlap. */
typedef struct {
    int32_t n_experts;   /* E, 1..1024 */
    int32_t n_ranks;     /* R, 1..64, divides E */
    int32_t window;      /* forwards in the sliding window, 1..4096 */
    int32_t max_moves;   /* copies added per triggered rebalance, 0..64 */
    int32_t spare_slots; /* extra slots per rank for added copies, 0..64 */
    double threshold;    /* trigger: max / mean rank load > threshold (>= 1) */
} moe_eplb_config;

/* Per-expert token counts of one forward: counts[e] = #{(t, k): topk_idx[t][k]
 * == e}, e < E (int32 [E], overwritten; ids outside [0, E) are ignored).
 * Exact (integer) and independent of the order of the additions. */
moe_status moe_expert_counts(const moe_shape *shape, int32_t T, const int32_t *topk_idx,
                             int32_t *counts, void *stream);

/* (host) Bytes of monitor state for cfg; 0 if cfg is invalid. */
size_t moe_eplb_state_bytes(const moe_eplb_config *cfg);
/* (host) Initialise the state: empty window, one home copy per expert. */
moe_status moe_eplb_init(const moe_eplb_config *cfg, void *state, size_t state_bytes);
/* (host) Push one forward's counts (host int32 [E], each >= 0). */
moe_status moe_eplb_observe(void *state, const int32_t *counts);
/* (host) Rank loads over the window (double [R], may be NULL) and max/mean
 * (0 when every load is 0). */
moe_status moe_eplb_loads(const void *state, double *loads, double *imbalance);
/* (host) If max/mean > threshold, add up to max_moves copies; *n_moves gets
 * the number added and moves (int32 [max_moves][2], may be NULL) the
 * (expert, rank) pairs in order.  No trigger: *n_moves = 0. */
moe_status moe_eplb_rebalance(void *state, int32_t *n_moves, int32_t *moves);
/* (host) One rank's table: rep_off [E+1], rep_slot [E + R * spare_slots],
 * slot_expert [E/R + spare_slots] (may be NULL: the expert each local slot
 * must hold, -1 for a reclaimed or empty slot), *n_slots (may be NULL). */
moe_status moe_eplb_slot_map(const void *state, int32_t rank, int32_t *rep_off,
                             int32_t *rep_slot, int32_t *slot_expert, int32_t *n_slots);
/* (host) Step 4: reclaim the original-position copies of the migrations
 * since the last cleanup (see above), in expert order then rank order.
 * *n_reclaimed gets the number reclaimed; the first `capacity` of them are
 * written to reclaimed (int32 [capacity][3]: expert, rank, local slot on
 * that rank whose weights may now be released; may be NULL if capacity is
 * 0).  At most E * R copies are reclaimed by one call. */
moe_status moe_eplb_cleanup(void *state, int32_t capacity, int32_t *n_reclaimed,
                            int32_t *reclaimed);

/* (host) Workspace bytes that moe_layer_forward needs for T tokens; also
 * enough for moe_dispatch and moe_expert_ffn with cap_rows <= T*K (or
 * n_shared*T for the shared experts).  Returns 0 for an invalid shape. */
size_t moe_workspace_bytes(const moe_shape *shape, int32_t T);

/* (host) Static string naming a status. */
const char *moe_status_str(moe_status status);

/* (host) Library version, "major.minor.patch". */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
