// eplb.cpp -- EPLB-lite: the host side of the expert-parallelism blog page's
// section 6.2 load balancer, with the redundant copies of section 6.3.
//
//   monitor   a sliding window of per-forward expert counts (the device
//             histogram moe_expert_counts feeds it); a rank's load is the
//             sum of count_e / n_copies_e over the copies it holds
//   detect    max(rank load) / mean(rank load) > threshold (1.2 on the page)
//   migrate   greedy: on the most loaded rank take the copy with the largest
//             per-copy load that can still be placed, add a copy on the least
//             loaded rank that lacks one and has a spare slot; repeat up to
//             max_moves times (the page: the hottest one or two experts)
//   tables    per-rank expert -> slot lists (moe_slot_map layout) for the
//             current placement; the caller keeps two device copies and
//             switches between forwards (the page's double-buffered routing
//             table: work already queued keeps reading the old one)
//   cleanup   once the old table has drained, the copy each migration was
//             taken from (its original position) is reclaimed, so the
//             migration becomes a move; a reclaimed home slot stays empty, a
//             reclaimed spare slot becomes a hole the next copy fills
//
// All state lives in caller memory (moe_eplb_state_bytes); nothing here
// touches a device.  Loads are double sums accumulated in expert order, so
// every decision is reproducible.
#include <math.h>
#include <string.h>

#include "moe.h"

namespace {

constexpr int kMaxRanks = 64;
constexpr int kMaxWindow = 4096;
constexpr int kMaxSpare = 64;

struct Hdr {
    moe_eplb_config cfg;
    int32_t filled;  // histograms in the window (<= W)
    int32_t head;    // next ring slot to write
};

struct View {
    Hdr *h;
    int32_t *ring;       // [W][E]
    int64_t *sum;        // [E] window sums
    int32_t *ncopy;      // [E]
    int32_t *copies;     // [E][R]: ranks holding a copy, in creation order
    int32_t *nadded;     // [R]: spare slots in use or holes
    int32_t *added;      // [R][spare]: expert in each spare slot, -1 = hole
    int32_t *home_live;  // [E]: the home copy has not been reclaimed
    uint8_t *pend;       // [E][R]: a migration took e from rank r since the last cleanup
};

size_t align8(size_t n) { return (n + 7) & ~(size_t)7; }

constexpr int kParts = 8;

size_t layout(const moe_eplb_config &c, size_t *off) {
    size_t o = align8(sizeof(Hdr));
    off[0] = o;
    o += align8((size_t)c.window * c.n_experts * 4);
    off[1] = o;
    o += (size_t)c.n_experts * 8;
    off[2] = o;
    o += align8((size_t)c.n_experts * 4);
    off[3] = o;
    o += align8((size_t)c.n_experts * c.n_ranks * 4);
    off[4] = o;
    o += align8((size_t)c.n_ranks * 4);
    off[5] = o;
    o += align8((size_t)c.n_ranks * (c.spare_slots > 0 ? c.spare_slots : 1) * 4);
    off[6] = o;
    o += align8((size_t)c.n_experts * 4);
    off[7] = o;
    o += align8((size_t)c.n_experts * c.n_ranks);
    return o;
}

bool valid(const moe_eplb_config *c) {
    return c && c->n_experts >= 1 && c->n_experts <= 1024 && c->n_ranks >= 1 &&
           c->n_ranks <= kMaxRanks && c->n_experts % c->n_ranks == 0 && c->window >= 1 &&
           c->window <= kMaxWindow && c->max_moves >= 0 && c->max_moves <= 64 &&
           c->spare_slots >= 0 && c->spare_slots <= kMaxSpare && c->threshold >= 1.0 &&
           isfinite(c->threshold);
}

template <typename S>
View view(S *state) {
    char *b = (char *)state;
    View v;
    v.h = (Hdr *)b;
    size_t off[kParts];
    layout(v.h->cfg, off);
    v.ring = (int32_t *)(b + off[0]);
    v.sum = (int64_t *)(b + off[1]);
    v.ncopy = (int32_t *)(b + off[2]);
    v.copies = (int32_t *)(b + off[3]);
    v.nadded = (int32_t *)(b + off[4]);
    v.added = (int32_t *)(b + off[5]);
    v.home_live = (int32_t *)(b + off[6]);
    v.pend = (uint8_t *)(b + off[7]);
    return v;
}

int spare_stride(const moe_eplb_config &c) { return c.spare_slots > 0 ? c.spare_slots : 1; }

// First free spare slot of rank r: a hole, else the next unused one; -1
// when every spare slot holds a copy.
int free_spare(const View &v, int r) {
    const moe_eplb_config &c = v.h->cfg;
    const int sp = spare_stride(c);
    for (int j = 0; j < v.nadded[r]; ++j)
        if (v.added[r * sp + j] < 0) return j;
    return v.nadded[r] < c.spare_slots ? v.nadded[r] : -1;
}

bool holds(const View &v, int e, int r) {
    const int R = v.h->cfg.n_ranks;
    for (int i = 0; i < v.ncopy[e]; ++i)
        if (v.copies[e * R + i] == r) return true;
    return false;
}

void compute_loads(const View &v, double *load) {
    const int E = v.h->cfg.n_experts, R = v.h->cfg.n_ranks;
    for (int r = 0; r < R; ++r) load[r] = 0.0;
    for (int e = 0; e < E; ++e) {
        const double share = (double)v.sum[e] / (double)v.ncopy[e];
        for (int i = 0; i < v.ncopy[e]; ++i) load[v.copies[e * R + i]] += share;
    }
}

double imbalance_of(const double *load, int R) {
    double tot = 0.0, mx = load[0];
    for (int r = 0; r < R; ++r) {
        tot += load[r];
        if (load[r] > mx) mx = load[r];
    }
    const double mean = tot / R;
    return mean > 0.0 ? mx / mean : 0.0;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) size_t moe_eplb_state_bytes(const moe_eplb_config *cfg) {
    if (!valid(cfg)) return 0;
    size_t off[kParts];
    return layout(*cfg, off);
}

__attribute__((visibility("default"))) moe_status moe_eplb_init(const moe_eplb_config *cfg,
                                                                void *state, size_t state_bytes) {
    if (!valid(cfg)) return MOE_ERR_SHAPE;
    if (!state) return MOE_ERR_INVALID_ARG;
    size_t off[kParts];
    const size_t need = layout(*cfg, off);
    if (state_bytes < need) return MOE_ERR_WORKSPACE;
    memset(state, 0, need);
    View v = view(state);
    v.h->cfg = *cfg;
    const int E = cfg->n_experts, R = cfg->n_ranks, per = E / R;
    v = view(state);
    for (int e = 0; e < E; ++e) {
        v.ncopy[e] = 1;
        v.copies[e * R] = e / per;  // home copy, section 2.1 placement
        v.home_live[e] = 1;
    }
    return MOE_OK;
}

__attribute__((visibility("default"))) moe_status moe_eplb_observe(void *state,
                                                                   const int32_t *counts) {
    if (!state || !counts) return MOE_ERR_INVALID_ARG;
    View v = view(state);
    const moe_eplb_config &c = v.h->cfg;
    const int E = c.n_experts;
    for (int e = 0; e < E; ++e)
        if (counts[e] < 0) return MOE_ERR_INVALID_ARG;
    int32_t *slot = v.ring + (size_t)v.h->head * E;
    if (v.h->filled == c.window)
        for (int e = 0; e < E; ++e) v.sum[e] -= slot[e];  // the oldest forward leaves
    else
        v.h->filled += 1;
    for (int e = 0; e < E; ++e) {
        slot[e] = counts[e];
        v.sum[e] += counts[e];
    }
    v.h->head = (v.h->head + 1) % c.window;
    return MOE_OK;
}

__attribute__((visibility("default"))) moe_status moe_eplb_loads(const void *state, double *loads,
                                                                 double *imbalance) {
    if (!state) return MOE_ERR_INVALID_ARG;
    View v = view(state);
    double load[kMaxRanks];
    compute_loads(v, load);
    const int R = v.h->cfg.n_ranks;
    if (loads)
        for (int r = 0; r < R; ++r) loads[r] = load[r];
    if (imbalance) *imbalance = imbalance_of(load, R);
    return MOE_OK;
}

__attribute__((visibility("default"))) moe_status moe_eplb_rebalance(void *state,
                                                                     int32_t *n_moves,
                                                                     int32_t *moves) {
    if (!state || !n_moves) return MOE_ERR_INVALID_ARG;
    View v = view(state);
    const moe_eplb_config &c = v.h->cfg;
    const int E = c.n_experts, R = c.n_ranks;
    *n_moves = 0;
    double load[kMaxRanks];
    compute_loads(v, load);
    if (!(imbalance_of(load, R) > c.threshold)) return MOE_OK;
    for (int m = 0; m < c.max_moves; ++m) {
        compute_loads(v, load);
        int hot = 0;
        for (int r = 1; r < R; ++r)
            if (load[r] > load[hot]) hot = r;  // ties: lower rank
        // candidates on the hot rank in (per-copy load desc, id asc) order:
        // repeatedly take the best not yet tried
        bool placed = false;
        uint8_t tried[1024] = {0};
        for (;;) {
            int best = -1;
            double bval = 0.0;
            for (int e = 0; e < E; ++e) {
                if (tried[e] || !holds(v, e, hot)) continue;
                const double per_copy = (double)v.sum[e] / (double)v.ncopy[e];
                if (best < 0 || per_copy > bval) {
                    best = e;
                    bval = per_copy;
                }
            }
            if (best < 0) break;
            tried[best] = 1;
            int tgt = -1;
            for (int r = 0; r < R; ++r) {
                if (holds(v, best, r) || free_spare(v, r) < 0) continue;
                if (tgt < 0 || load[r] < load[tgt]) tgt = r;  // ties: lower rank
            }
            if (tgt < 0) continue;
            v.copies[best * R + v.ncopy[best]] = tgt;
            v.ncopy[best] += 1;
            const int j = free_spare(v, tgt);
            v.added[tgt * spare_stride(c) + j] = best;
            if (j == v.nadded[tgt]) v.nadded[tgt] += 1;
            v.pend[best * R + hot] = 1;  // the copy this migration was taken from
            if (moves) {
                moves[2 * *n_moves] = best;
                moves[2 * *n_moves + 1] = tgt;
            }
            *n_moves += 1;
            placed = true;
            break;
        }
        if (!placed) break;
    }
    return MOE_OK;
}

__attribute__((visibility("default"))) moe_status moe_eplb_slot_map(
    const void *state, int32_t rank, int32_t *rep_off, int32_t *rep_slot, int32_t *slot_expert,
    int32_t *n_slots) {
    if (!state || !rep_off || !rep_slot) return MOE_ERR_INVALID_ARG;
    View v = view(state);
    const moe_eplb_config &c = v.h->cfg;
    const int E = c.n_experts, R = c.n_ranks, per = E / R;
    const int sp = c.spare_slots > 0 ? c.spare_slots : 1;
    if (rank < 0 || rank >= R) return MOE_ERR_SHAPE;
    const int S = per + v.nadded[rank];
    if (slot_expert) {
        for (int s = 0; s < per; ++s)
            slot_expert[s] = v.home_live[rank * per + s] ? rank * per + s : -1;
        for (int j = 0; j < v.nadded[rank]; ++j) slot_expert[per + j] = v.added[rank * sp + j];
    }
    if (n_slots) *n_slots = S;
    int n = 0;
    rep_off[0] = 0;
    for (int e = 0; e < E; ++e) {
        for (int i = 0; i < v.ncopy[e]; ++i) {
            int s = -1;
            if (v.copies[e * R + i] == rank) {
                if (e / per == rank && v.home_live[e]) {
                    s = e - rank * per;
                } else {
                    for (int j = 0; j < v.nadded[rank]; ++j)
                        if (v.added[rank * sp + j] == e) s = per + j;
                }
            }
            rep_slot[n++] = s;
        }
        rep_off[e + 1] = n;
    }
    return MOE_OK;
}

__attribute__((visibility("default"))) moe_status moe_eplb_cleanup(void *state,
                                                                   int32_t capacity,
                                                                   int32_t *n_reclaimed,
                                                                   int32_t *reclaimed) {
    if (!state || !n_reclaimed || capacity < 0 || (capacity > 0 && !reclaimed))
        return MOE_ERR_INVALID_ARG;
    View v = view(state);
    const moe_eplb_config &c = v.h->cfg;
    const int E = c.n_experts, R = c.n_ranks, per = E / R, sp = spare_stride(c);
    int n = 0;
    for (int e = 0; e < E; ++e) {
        for (int r = 0; r < R; ++r) {
            if (!v.pend[e * R + r]) continue;
            v.pend[e * R + r] = 0;
            if (!holds(v, e, r) || v.ncopy[e] < 2) continue;  // keep the last copy
            int slot = -1;
            if (e / per == r && v.home_live[e]) {
                slot = e - r * per;
                v.home_live[e] = 0;
            } else {
                for (int j = 0; j < v.nadded[r]; ++j)
                    if (v.added[r * sp + j] == e) {
                        slot = per + j;
                        v.added[r * sp + j] = -1;
                    }
            }
            int w = 0;  // drop r from e's copies, keeping the others' order
            for (int i = 0; i < v.ncopy[e]; ++i)
                if (v.copies[e * R + i] != r) v.copies[e * R + w++] = v.copies[e * R + i];
            v.ncopy[e] = w;
            if (n < capacity) {
                reclaimed[3 * n] = e;
                reclaimed[3 * n + 1] = r;
                reclaimed[3 * n + 2] = slot;
            }
            ++n;
        }
    }
    *n_reclaimed = n;
    return MOE_OK;
}

}  // extern "C"
