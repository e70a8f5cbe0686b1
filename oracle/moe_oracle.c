/*
 * moe_oracle.c -- plain CPU oracle for one DeepSeek-V3-style MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may build, load or call this file.  The HIP
 * path shares no code, header, table or constant with it.
 *
 * What it computes follows the expert-parallelism blog page (yveltals,
 * "专家并行（EP）"): section 2.2 walks one token through the layer in five
 * steps (router linear + top-8, dispatch, expert FFN, combine, weighted sum
 * plus the shared expert); section 2.1 gives the contiguous expert placement
 * and the two replicated shared experts; section 6.3 gives redundant expert
 * replicas chosen at random.  Where the page leaves a step open this file
 * takes the reading written at each function.
 *
 * Conventions: every dot product accumulates in double; every stored value
 * is float.  Inputs are fp16 (IEEE binary16 bit patterns) or fp32, chosen by
 * a dtype flag; fp16 values are decoded exactly.  Loops are plain and
 * single-threaded; loop nests are ordered for cache reuse only (each dot
 * product is still evaluated on its own, index ascending).
 *
 * Parity pins (tests/test_oracle_pins.py) check every function here against
 * closed forms, brute force on small inputs, and the page's worked example.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OREF_F32 = 0, OREF_F16 = 1 };

/* ------------------------------------------------------------------ */
/* Input decoding                                                      */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; exponent 0 encodes zero/subnormals (f * 2^-24), 31 encodes inf/NaN. */
double oref_f16_to_double(uint16_t b)
{
    int s = (b >> 15) & 1, e = (b >> 10) & 0x1f, f = b & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

static double g_f16tab[65536];
static int g_f16tab_ready = 0;

static void f16tab_init(void)
{
    if (g_f16tab_ready)
        return;
    for (int i = 0; i < 65536; ++i)
        g_f16tab[i] = oref_f16_to_double((uint16_t)i);
    g_f16tab_ready = 1;
}

static inline double in_at(const void *p, int dtype, size_t i)
{
    if (dtype == OREF_F16)
        return g_f16tab[((const uint16_t *)p)[i]];
    return (double)((const float *)p)[i];
}

/* Plain dot product of row a (length n, dtype) with a double vector x. */
static double dot_in(const void *a, int dtype, size_t off, const double *x, int n)
{
    double acc = 0.0;
    for (int i = 0; i < n; ++i)
        acc += in_at(a, dtype, off + (size_t)i) * x[i];
    return acc;
}

static void load_row(const void *h, int dtype, size_t off, int n, double *x)
{
    for (int i = 0; i < n; ++i)
        x[i] = in_at(h, dtype, off + (size_t)i);
}

/* ------------------------------------------------------------------ */
/* Step 1: router linear and top-K (blog section 2.2, Step 1)          */
/* ------------------------------------------------------------------ */

/* logits[t][e] = fp32( sum_i h[t][i] * Wr[e][i] ) + bias[e]
 * The page's router maps a [1, 7168] hidden row through a [7168, 256]
 * linear to [1, 256] logits.  Wr is stored row per expert ([E][H]); the
 * optional bias (fp32, added in fp32 after rounding the sum) is how the
 * long-tail workloads skew routing. */
void oref_router_logits(int T, int H, int E, int dtype, const void *h,
                        const void *w_router, const float *bias, float *logits)
{
    f16tab_init();
    double *x = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    for (int t = 0; t < T; ++t) {
        load_row(h, dtype, (size_t)t * H, H, x);
        for (int e = 0; e < E; ++e) {
            float l = (float)dot_in(w_router, dtype, (size_t)e * H, x, H);
            if (bias)
                l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
    }
    free(x);
}

/* Step 1 (top-K) and Step 5 (gate weights).
 * The page picks K = 8 experts per token and weights expert i's output by
 * softmax(logits)[i].  Reading taken: the softmax runs over all E logits and
 * the K selected probabilities are used as they are (not renormalised);
 * selection orders experts by logit, larger first, and the lower id wins a
 * tie.  topk_idx[t][0..K-1] lists the winners in that order. */
/* Group-limited top-K: the large-EP outlook of the expert-parallelism blog
 * page (section 八) routes to groups of experts first, then to experts
 * inside the chosen groups.  Reading taken: G contiguous groups of E/G
 * experts (the contiguous placement of section 2.1, so a group is one EP
 * rank); a group's score is its largest logit; the M groups with the
 * largest scores are kept (ties: lower group id); the K experts are then
 * picked among the kept groups' experts exactly as above; gates stay the
 * softmax over all E logits.  G == 0 means no group limit. */
void oref_softmax_topk_grouped(int T, int E, int K, int G, int M, const float *logits,
                               int32_t *topk_idx, float *topk_w);

void oref_softmax_topk(int T, int E, int K, const float *logits,
                       int32_t *topk_idx, float *topk_w)
{
    oref_softmax_topk_grouped(T, E, K, 0, 0, logits, topk_idx, topk_w);
}

void oref_softmax_topk_grouped(int T, int E, int K, int G, int M, const float *logits,
                               int32_t *topk_idx, float *topk_w)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            z += p[e];
        }
        for (int e = 0; e < E; ++e)
            p[e] /= z;
        memset(taken, 0, (size_t)E);
        if (G > 0) {
            /* pick M groups by their best logit; experts of the other
             * groups are marked taken so the expert rounds skip them */
            const int gs = E / G;
            char *gsel = (char *)calloc((size_t)G, 1);
            for (int r = 0; r < M; ++r) {
                int bg = -1;
                float bs = 0.0f;
                for (int g = 0; g < G; ++g) {
                    if (gsel[g])
                        continue;
                    float sc = l[g * gs];
                    for (int e = g * gs + 1; e < (g + 1) * gs; ++e)
                        if (l[e] > sc)
                            sc = l[e];
                    if (bg < 0 || sc > bs) { /* strict '>': lower group id on ties */
                        bg = g;
                        bs = sc;
                    }
                }
                gsel[bg] = 1;
            }
            for (int e = 0; e < E; ++e)
                if (!gsel[e / gs])
                    taken[e] = 1;
            free(gsel);
        }
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e; /* strict '>' keeps the lower id on ties */
            }
            taken[best] = 1;
            topk_idx[(size_t)t * K + k] = best;
            topk_w[(size_t)t * K + k] = (float)p[best];
        }
    }
    free(taken);
    free(p);
}

/* Step 5 shared-expert gate.  The page multiplies the shared experts'
 * output by a gate without saying what the gate is; reading taken:
 * gate[t] = sigmoid(h[t] . w_sg) with one learned vector w_sg, the dot
 * product rounded to fp32 like a router logit. */
void oref_shared_gate(int T, int H, int dtype, const void *h, const void *w_sg,
                      float *gate)
{
    f16tab_init();
    double *x = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    for (int t = 0; t < T; ++t) {
        load_row(h, dtype, (size_t)t * H, H, x);
        float z = (float)dot_in(w_sg, dtype, 0, x, H);
        gate[t] = (float)(1.0 / (1.0 + exp(-(double)z)));
    }
    free(x);
}

/* ------------------------------------------------------------------ */
/* Expert -> local slot (blog sections 2.1 and 6.3)                    */
/* ------------------------------------------------------------------ */

/* SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): add the golden-gamma
 * increment, then two xor-shift-multiply rounds and a final xor-shift. */
uint64_t oref_splitmix64(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* slot[t][k] for expert e = topk_idx[t][k]: the replicas of e are
 * rep_slot[rep_off[e] .. rep_off[e+1]) (a local slot, or -1 when that copy
 * lives on another GPU).  Section 6.3 sends a token to a random replica;
 * reading taken: the choice is replica number
 * splitmix64(seed ^ (tok*K + k)) mod n_replicas, where tok is the token's
 * index in the batch (tok_ids[t] if given, else t). */
void oref_slot_map(int T, int K, const int32_t *topk_idx, const int32_t *tok_ids,
                   const int32_t *rep_off, const int32_t *rep_slot, uint64_t seed,
                   int32_t *slot)
{
    for (int t = 0; t < T; ++t) {
        uint64_t tok = (uint64_t)(tok_ids ? tok_ids[t] : t);
        for (int k = 0; k < K; ++k) {
            int e = topk_idx[(size_t)t * K + k];
            int n = rep_off[e + 1] - rep_off[e];
            int r = 0;
            if (n > 1)
                r = (int)(oref_splitmix64(seed ^ (tok * (uint64_t)K + (uint64_t)k)) %
                          (uint64_t)n);
            slot[(size_t)t * K + k] = n > 0 ? rep_slot[rep_off[e] + r] : -1;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 2: dispatch (blog section 2.2, Step 2)                          */
/* ------------------------------------------------------------------ */

/* On one GPU the page's scatter becomes a permutation: every (t, k) whose
 * slot is local becomes one row of a per-slot contiguous group.  Reading
 * taken: groups in slot order, rows inside a group in token order, no
 * capacity limit and no dropped pairs.  This is a stable counting sort:
 *   counts[s]  = number of pairs with slot s
 *   offsets    = exclusive prefix sum of counts (offsets[S] = total rows)
 *   perm_src[row] = t*K + k of the pair that fills the row
 *   inv_pos[t*K + k] = its row, or -1 when the pair is not local. */
void oref_dispatch(int T, int K, int S, const int32_t *slot, int32_t *counts,
                   int32_t *offsets, int32_t *perm_src, int32_t *inv_pos)
{
    for (int s = 0; s < S; ++s)
        counts[s] = 0;
    for (size_t p = 0; p < (size_t)T * K; ++p)
        if (slot[p] >= 0)
            counts[slot[p]]++;
    offsets[0] = 0;
    for (int s = 0; s < S; ++s)
        offsets[s + 1] = offsets[s] + counts[s];
    int32_t *fill = (int32_t *)calloc((size_t)(S > 0 ? S : 1), sizeof(int32_t));
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            size_t p = (size_t)t * K + k;
            int s = slot[p];
            if (s < 0) {
                inv_pos[p] = -1;
                continue;
            }
            int row = offsets[s] + fill[s]++;
            inv_pos[p] = row;
            perm_src[row] = (int32_t)p;
        }
    free(fill);
}

/* ------------------------------------------------------------------ */
/* FP8 dispatch payload (blog section 2.3: FP8 halves the traffic)     */
/* ------------------------------------------------------------------ */

/* OCP 8-bit floating point, E4M3 (OFP8 specification rev 1.0): sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
 * subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN, so the largest
 * finite magnitude is 1.75 * 2^8 = 448.  Encoding rounds to nearest, ties to
 * even.  Input must already lie in [-448, 448]. */
uint8_t oref_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid, spacing 2^-9; m == 8 is the smallest normal */
        long m = lrint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int ex;
    double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;           /* a = (2f) * 2^E, 2f in [1, 2) */
    long m = lrint((2.0 * f - 1.0) * 8.0);
    if (m == 8) {
        m = 0;
        E += 1;
    }
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)m);
}

float oref_e4m3_decode(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 0xf, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return (float)(s ? -v : v);
}

/* Per-row symmetric quantisation (reading taken: one fp32 scale per token,
 * the row's absolute maximum mapped to 448):
 *   amax = max |x|;  inv = 448 / amax;  scale = amax / 448   (fp32, each
 *   a correctly rounded division);  q = E4M3(clamp(x * inv, -448, 448)).
 * An all-zero row gets scale 0 and codes 0. */
void oref_quant_e4m3_rows(int R, int H, int dtype, const void *x, uint8_t *q,
                          float *scale)
{
    f16tab_init();
    for (int r = 0; r < R; ++r) {
        float amax = 0.0f;
        for (int i = 0; i < H; ++i) {
            float a = fabsf((float)in_at(x, dtype, (size_t)r * H + i));
            if (a > amax)
                amax = a;
        }
        if (amax == 0.0f) {
            scale[r] = 0.0f;
            memset(q + (size_t)r * H, 0, (size_t)H);
            continue;
        }
        volatile float inv = 448.0f / amax;
        scale[r] = amax / 448.0f;
        for (int i = 0; i < H; ++i) {
            volatile float v = (float)in_at(x, dtype, (size_t)r * H + i) * inv;
            float c = v;
            if (c > 448.0f)
                c = 448.0f;
            if (c < -448.0f)
                c = -448.0f;
            q[(size_t)r * H + i] = oref_e4m3_encode(c);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 3: expert FFN (blog section 2.2 Step 3; section 一 gives the    */
/* gate/up shape [7168, 2048]; section 6.3's 88 MB per expert implies  */
/* a third matrix of the same size, the down projection [2048, 7168]) */
/* ------------------------------------------------------------------ */

/* SwiGLU expert on R rows x[r] (double values):
 *   a = Wg x, b = Wu x                 (Wg, Wu stored [I][H])
 *   hm = fp32( silu(a) * b ),  silu(z) = z / (1 + exp(-z))
 *   y  = fp32( Wd hm )                 (Wd stored [H][I])
 * hm may be NULL. */
void oref_expert_rows(int R, int H, int I, int dtype, const double *x,
                      const void *wg, const void *wu, const void *wd,
                      float *hm, float *y)
{
    f16tab_init();
    double *a = (double *)malloc(sizeof(double) * (size_t)R * I);
    for (int i = 0; i < I; ++i)
        for (int r = 0; r < R; ++r) {
            double ga = dot_in(wg, dtype, (size_t)i * H, x + (size_t)r * H, H);
            double ub = dot_in(wu, dtype, (size_t)i * H, x + (size_t)r * H, H);
            double silu = ga / (1.0 + exp(-ga));
            a[(size_t)r * I + i] = (double)(float)(silu * ub);
        }
    if (hm)
        for (size_t j = 0; j < (size_t)R * I; ++j)
            hm[j] = (float)a[j];
    for (int o = 0; o < H; ++o)
        for (int r = 0; r < R; ++r)
            y[(size_t)r * H + o] = (float)dot_in(wd, dtype, (size_t)o * I,
                                                 a + (size_t)r * I, I);
    free(a);
}

/* ------------------------------------------------------------------ */
/* Steps 4 and 5: combine and weighted sum (blog section 2.2)          */
/* ------------------------------------------------------------------ */

/* out[t] = sum over k (in k order) of topk_w[t][k] * y[inv_pos[t][k]]
 *          (pairs with inv_pos = -1 are computed elsewhere and skipped)
 *        + shared_gate[t] * sum_j shared_y[j][t]     (if shared_y given)
 * accumulated in double, stored fp32. */
void oref_combine(int T, int K, int H, int n_shared, const float *y,
                  const int32_t *inv_pos, const float *topk_w,
                  const float *shared_y, const float *shared_gate, float *out)
{
    for (int t = 0; t < T; ++t)
        for (int o = 0; o < H; ++o) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                int r = inv_pos[(size_t)t * K + k];
                if (r >= 0)
                    acc += (double)topk_w[(size_t)t * K + k] * (double)y[(size_t)r * H + o];
            }
            if (shared_y && n_shared > 0) {
                double sh = 0.0;
                for (int j = 0; j < n_shared; ++j)
                    sh += (double)shared_y[((size_t)j * T + t) * H + o];
                acc += (double)shared_gate[t] * sh;
            }
            out[(size_t)t * H + o] = (float)acc;
        }
}

/* ------------------------------------------------------------------ */
/* The whole layer (Steps 1-5)                                         */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t T, H, I, E, K, S, n_shared, dtype, fp8_dispatch;
    int32_t n_groups, topk_groups; /* group-limited routing (0: none) */
} oref_dims;

/* One MoE layer forward for T tokens.
 *   h [T][H]; w_router [E][H]; bias [E] or NULL; w_sg [H] (needed iff
 *   n_shared > 0); slot_gate/up/down: S pointers to each local slot's
 *   matrices ([I][H], [I][H], [H][I]; a NULL pointer means the slot's
 *   weights were not supplied, which is an error if a pair lands there);
 *   sh_gate/up/down [n_shared][..]; rep_off/rep_slot/seed: the slot map;
 *   tok_ids: batch index of each row of h (NULL = 0..T-1), used by the
 *   replica choice so a sample of tokens reproduces the full batch.
 * Outputs (each optional except out): out [T][H]; topk_idx, topk_w,
 * slot [T][K]; logits [T][E]; shared_gate [T].
 * Returns 0, or -1 if a pair needs a slot whose weights are missing. */
int oref_layer_forward(const oref_dims *d, const void *h, const int32_t *tok_ids,
                       const void *w_router, const float *bias, const void *w_sg,
                       const void *const *slot_gate, const void *const *slot_up,
                       const void *const *slot_down, const void *sh_gate,
                       const void *sh_up, const void *sh_down, const int32_t *rep_off,
                       const int32_t *rep_slot, uint64_t seed, float *out,
                       int32_t *topk_idx_out, float *topk_w_out, int32_t *slot_out,
                       float *logits_out, float *shared_gate_out)
{
    const int T = d->T, H = d->H, I = d->I, E = d->E, K = d->K, S = d->S;
    f16tab_init();
    float *logits = (float *)malloc(sizeof(float) * (size_t)T * E + 1);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * K + 1);
    float *w = (float *)malloc(sizeof(float) * (size_t)T * K + 1);
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * K + 1);
    int rc = 0;

    oref_router_logits(T, H, E, d->dtype, h, w_router, bias, logits);
    oref_softmax_topk_grouped(T, E, K, d->n_groups, d->topk_groups, logits, idx, w);
    oref_slot_map(T, K, idx, tok_ids, rep_off, rep_slot, seed, slot);

    /* A token's K experts are distinct (Step 1 picks K different experts)
     * and a slot holds one expert's weights, so no slot receives a token
     * twice and a slot holds at most T rows.  Inputs that break this (a
     * slot table listing one slot under two experts) are refused. */
    for (int t = 0; t < T && rc == 0; ++t)
        for (int k = 1; k < K && rc == 0; ++k)
            for (int j = 0; j < k; ++j)
                if (slot[(size_t)t * K + k] >= 0 &&
                    slot[(size_t)t * K + k] == slot[(size_t)t * K + j])
                    rc = -2;

    for (size_t j = 0; j < (size_t)T * H; ++j)
        out[j] = 0.0f;
    double *acc = (double *)calloc((size_t)T * H + 1, sizeof(double));

    /* routed experts, slot-outer so each slot's weights are walked once */
    /* a slot receives each token at most once (checked above), so R <= T */
    double *x = (double *)malloc(sizeof(double) * (size_t)T * H + 1);
    float *y = (float *)malloc(sizeof(float) * (size_t)T * H + 1);
    int32_t *pair = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * K + 1);
    uint8_t *q = (uint8_t *)malloc((size_t)H + 1);
    for (int s = 0; s < S && rc == 0; ++s) {
        int R = 0;
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k)
                if (slot[(size_t)t * K + k] == s)
                    pair[R++] = t * K + k;
        if (R == 0)
            continue;
        if (!slot_gate[s] || !slot_up[s] || !slot_down[s]) {
            rc = -1;
            break;
        }
        for (int r = 0; r < R; ++r) {
            int t = pair[r] / K;
            if (d->fp8_dispatch) {
                float sc;
                oref_quant_e4m3_rows(1, H, d->dtype, (const char *)h +
                                     (size_t)t * H * (d->dtype == OREF_F16 ? 2 : 4),
                                     q, &sc);
                for (int i = 0; i < H; ++i)
                    x[(size_t)r * H + i] = (double)(oref_e4m3_decode(q[i]) * sc);
            } else {
                load_row(h, d->dtype, (size_t)t * H, H, x + (size_t)r * H);
            }
        }
        oref_expert_rows(R, H, I, d->dtype, x, slot_gate[s], slot_up[s],
                         slot_down[s], NULL, y);
        for (int r = 0; r < R; ++r) {
            int t = pair[r] / K;
            double g = (double)w[pair[r]];
            for (int o = 0; o < H; ++o)
                acc[(size_t)t * H + o] += g * (double)y[(size_t)r * H + o];
        }
    }
    /* The per-token sums run slot by slot rather than k by k; they are
     * double sums of fp32 terms, so the order cannot change the fp32 result
     * beyond one rounding of the final conversion. */

    /* shared experts (every token, Step 5) */
    float *gs = (float *)malloc(sizeof(float) * (size_t)T + 1);
    if (rc == 0 && d->n_shared > 0) {
        oref_shared_gate(T, H, d->dtype, h, w_sg, gs);
        for (int t = 0; t < T; ++t)
            load_row(h, d->dtype, (size_t)t * H, H, x + (size_t)t * H);
        size_t isz = d->dtype == OREF_F16 ? 2 : 4;
        double *shsum = (double *)calloc((size_t)T * H + 1, sizeof(double));
        for (int j = 0; j < d->n_shared; ++j) {
            oref_expert_rows(T, H, I, d->dtype, x,
                             (const char *)sh_gate + (size_t)j * I * H * isz,
                             (const char *)sh_up + (size_t)j * I * H * isz,
                             (const char *)sh_down + (size_t)j * H * I * isz, NULL, y);
            for (size_t n = 0; n < (size_t)T * H; ++n)
                shsum[n] += (double)y[n];
        }
        for (int t = 0; t < T; ++t)
            for (int o = 0; o < H; ++o)
                acc[(size_t)t * H + o] += (double)gs[t] * shsum[(size_t)t * H + o];
        free(shsum);
    }
    if (rc == 0)
        for (size_t n = 0; n < (size_t)T * H; ++n)
            out[n] = (float)acc[n];

    if (topk_idx_out)
        memcpy(topk_idx_out, idx, sizeof(int32_t) * (size_t)T * K);
    if (topk_w_out)
        memcpy(topk_w_out, w, sizeof(float) * (size_t)T * K);
    if (slot_out)
        memcpy(slot_out, slot, sizeof(int32_t) * (size_t)T * K);
    if (logits_out)
        memcpy(logits_out, logits, sizeof(float) * (size_t)T * E);
    if (shared_gate_out && d->n_shared > 0)
        memcpy(shared_gate_out, gs, sizeof(float) * (size_t)T);

    free(gs);
    free(q);
    free(pair);
    free(y);
    free(x);
    free(acc);
    free(slot);
    free(w);
    free(idx);
    free(logits);
    return rc;
}
