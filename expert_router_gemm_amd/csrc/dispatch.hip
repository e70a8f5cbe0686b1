// dispatch.hip -- Step 2 on one GPU: permute local (token, k) pairs into
// per-slot contiguous groups, optionally quantising rows to OCP E4M3.
//
// The expert-parallelism blog page (section 2.2, Step 2) sends each token's
// hidden row to the GPUs that own its experts; with one GPU holding this
// rank's share, the send becomes a stable permutation: rows grouped by local
// slot, token order inside a group, nothing dropped.  Slots come from the
// contiguous placement of section 2.1 and, for redundant experts, a random
// replica (section 6.3) chosen by a counter hash so the result is exact.
// Section 2.3 notes FP8 halves the dispatched bytes: with x_dtype = FP8 each
// row is stored as E4M3 codes with one fp32 scale.
//
// Decode-sized batches (T <= 1024 tokens, S <= 256 slots) run steps 1-3's
// index work in a single 1024-thread block.  Larger batches use three
// kernels.  All deterministic (no order-dependent atomics):
//  1. rank:    one wave per 64-token chunk.  Each (token, k) sets its lane bit
//              in a per-slot 64-bit LDS mask (an OR, so arrival order cannot
//              matter); the pair's rank inside the chunk is the popcount of
//              the mask bits of lower lanes, the chunk's count the popcount.
//  2. scan:    per slot, exclusive scan over chunks; then an exclusive scan
//              over slots gives offsets.  chunk_counts becomes chunk_base.
//  3. index:   one thread per pair: row = chunk_base + rank -> inv_pos,
//              perm_src.
// When the rows are materialised (x_perm given: fp8 codes, or a caller that
// wants the permuted copy) one block per token then reads its hidden row
// once and writes it, or its E4M3 codes and scale, to each of its local rows.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

__device__ __forceinline__ int slot_of(const DispatchArgs &a, int t, int k) {
    const int e = a.topk_idx[(size_t)t * a.K + k];
    if (e < 0 || e >= a.E) return -1;
    const int lo = a.rep_off[e];
    const int n = a.rep_off[e + 1] - lo;
    if (n <= 0) return -1;
    int r = 0;
    if (n > 1) r = (int)(splitmix64(a.seed ^ ((uint64_t)t * (uint64_t)a.K + (uint64_t)k)) % (uint64_t)n);
    const int s = a.rep_slot[lo + r];
    return (s >= 0 && s < a.S) ? s : -1;
}

// A token's pairs must land in distinct slots (its K experts are distinct,
// and a slot holds one expert).  Should two of them meet in one slot anyway
// (repeated ids in a caller's topk_idx, or a table listing a slot under two
// experts), the later pair is not dispatched: its slot becomes -1, so every
// row still belongs to exactly one pair and the result stays deterministic.
template <int KMAX>
__device__ __forceinline__ void drop_repeated_slots(int (&sl)[KMAX], int K = KMAX) {
#pragma unroll
    for (int k = 1; k < KMAX; ++k) {
        if (k >= K) continue;
#pragma unroll
        for (int j = 0; j < k; ++j)
            if (sl[k] >= 0 && sl[k] == sl[j]) sl[k] = -1;
    }
}

// Tickets of the down projection's fused combine: each of the token's
// feature tiles starts at its number of local pairs (slots after
// drop_repeated_slots, i.e. the rows it really gets).
__device__ __forceinline__ void seed_tickets(const DispatchArgs &a, int t, int np) {
    if (!a.tickets || t >= a.T) return;
    int32_t *tk = a.tickets + (size_t)t * a.n_tiles;
    for (int f = 0; f < a.n_tiles; ++f) tk[f] = np;
}

__global__ __launch_bounds__(256) void dispatch_rank_kernel(DispatchArgs a) {
    extern __shared__ unsigned long long masks[];  // [4][S]
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const int chunk = blockIdx.x * 4 + wave;
    const int C = (a.T + 63) / 64;
    unsigned long long *m = masks + (size_t)wave * a.S;
    for (int s = lane; s < a.S; s += 64) m[s] = 0ull;
    __syncthreads();
    const int t = chunk * 64 + lane;
    const unsigned long long bit = 1ull << lane;
    // the token's slots, kept in registers for the ranking pass (top_k <= 16)
    int sk[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) sk[k] = (t < a.T && k < a.K) ? slot_of(a, t, k) : -1;
    drop_repeated_slots<16>(sk);
    {
        int np = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) np += sk[k] >= 0;
        seed_tickets(a, t, np);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (sk[k] >= 0) atomicOr(&m[sk[k]], bit);
    __syncthreads();
    if (t < a.T)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (k >= a.K) break;
            const int s = sk[k];
            int code = -1;
            if (s >= 0) code = s * 64 + __popcll(m[s] & (bit - 1ull));
            a.pair_code[(size_t)t * a.K + k] = code;
        }
    if (chunk < C)
        for (int s = lane; s < a.S; s += 64) a.chunk_counts[(size_t)chunk * a.S + s] = __popcll(m[s]);
}

// Single block of 1024 threads; S <= 1024.  P = 1024 / SP threads serve
// each slot (SP = S rounded up to a power of two), thread j of a slot owning
// a contiguous run of chunks:
//  1. per thread: sum of its chunks' counts; exclusive scan over the slot's
//     threads (segmented Hillis-Steele in LDS) and the slot total;
//  2. exclusive scan of the slot totals over slots -> counts, offsets;
//  3. per thread: chunk_counts of its chunks become absolute row bases
//     (slot offset + rows of the slot's earlier chunks).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(DispatchArgs a) {
    __shared__ int buf[2][1024];
    __shared__ int slot_tot[1024];
    const int C = (a.T + 63) / 64;
    int SP = 1;
    while (SP < a.S) SP <<= 1;
    const int P = 1024 / SP;
    const int tid = threadIdx.x;
    const int s = tid / P, j = tid % P;
    const bool live = s < a.S;
    const int cpt = (C + P - 1) / P;
    const int c0 = min(C, j * cpt), c1 = min(C, c0 + cpt);
    int sum = 0;
    if (live) {
#pragma unroll 8
        for (int c = c0; c < c1; ++c) sum += a.chunk_counts[(size_t)c * a.S + s];
    }
    // 1. inclusive scan of the per-thread sums within each slot's P threads
    int cur = 0;
    buf[0][tid] = sum;
    __syncthreads();
    for (int o = 1; o < P; o <<= 1) {
        const int v = buf[cur][tid] + (j >= o ? buf[cur][tid - o] : 0);
        buf[cur ^ 1][tid] = v;
        cur ^= 1;
        __syncthreads();
    }
    const int excl_j = buf[cur][tid] - sum;
    if (j == P - 1) slot_tot[s] = buf[cur][tid];
    __syncthreads();
    // 2. exclusive scan of the slot totals (entries past S are 0)
    int cs = 0;
    if (tid < SP) buf[0][tid] = slot_tot[tid];
    __syncthreads();
    for (int o = 1; o < SP; o <<= 1) {
        if (tid < SP) buf[cs ^ 1][tid] = buf[cs][tid] + (tid >= o ? buf[cs][tid - o] : 0);
        cs ^= 1;
        __syncthreads();
    }
    if (tid < a.S) {
        const int inc = buf[cs][tid], tot = slot_tot[tid];
        a.counts[tid] = tot;
        a.offsets[tid] = inc - tot;
        if (tid == a.S - 1) a.offsets[a.S] = inc;
    }
    // 3. absolute row base of every chunk of this thread
    if (live) {
        int run = buf[cs][s] - slot_tot[s] + excl_j;
#pragma unroll 8
        for (int c = c0; c < c1; ++c) {
            const int v = a.chunk_counts[(size_t)c * a.S + s];
            a.chunk_counts[(size_t)c * a.S + s] = run;
            run += v;
        }
    }
}

// Index outputs of the large-batch path, one thread per (token, k) pair.
__global__ __launch_bounds__(256) void dispatch_index_kernel(DispatchArgs a) {
    const size_t p = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= (size_t)a.T * a.K) return;
    const int code = a.pair_code[p];
    if (code < 0) {
        a.inv_pos[p] = -1;
        return;
    }
    const int t = (int)(p / a.K);
    const int row = a.chunk_counts[(size_t)(t >> 6) * a.S + (code >> 6)] + (code & 63);
    a.inv_pos[p] = row;
    a.perm_src[row] = (int32_t)p;
}

// Large batches with a small (chunk, slot) table (S <= 256, C*S <= 64K):
// the scan and the index outputs in one launch, one block per chunk of 64
// tokens.  Each block re-derives, from the per-chunk counts, every slot's
// total and the rows its slot holds in earlier chunks (integer sums, so
// the order of the LDS atomics does not matter), scans the totals into
// slot offsets, and places its own pairs; block 0 writes counts and
// offsets.  Replaces dispatch_scan_kernel's single block and a launch.
constexpr int kPlaceMaxS = 256, kPlaceMaxTable = 65536;

__global__ __launch_bounds__(256) void dispatch_place_kernel(DispatchArgs a) {
    __shared__ int tot[kPlaceMaxS], before[kPlaceMaxS], scan[2][kPlaceMaxS];
    const int tid = threadIdx.x, c = blockIdx.x, S = a.S;
    const int C = (a.T + 63) / 64;
    if (tid < S) {
        tot[tid] = 0;
        before[tid] = 0;
    }
    __syncthreads();
    const int n = C * S;
    for (int i = tid; i < n; i += 256) {
        const int v = a.chunk_counts[i];
        const int sl = i % S;
        atomicAdd(&tot[sl], v);
        if (i / S < c) atomicAdd(&before[sl], v);
    }
    __syncthreads();
    // inclusive scan of the slot totals (entries past S are 0)
    int cur = 0;
    scan[0][tid] = tid < S ? tot[tid] : 0;
    __syncthreads();
    for (int o = 1; o < kPlaceMaxS; o <<= 1) {
        scan[cur ^ 1][tid] = scan[cur][tid] + (tid >= o ? scan[cur][tid - o] : 0);
        cur ^= 1;
        __syncthreads();
    }
    if (tid < S) {
        const int off = scan[cur][tid] - tot[tid];
        before[tid] += off;  // absolute first row of this chunk's pairs in slot tid
        if (c == 0) {
            a.counts[tid] = tot[tid];
            a.offsets[tid] = off;
            if (tid == S - 1) a.offsets[S] = scan[cur][tid];
        }
    }
    __syncthreads();
    const size_t p0 = (size_t)c * 64 * a.K;
    const size_t p1 = (size_t)min(a.T, (c + 1) * 64) * a.K;
    for (size_t p = p0 + tid; p < p1; p += 256) {
        const int code = a.pair_code[p];
        if (code < 0) {
            a.inv_pos[p] = -1;
            continue;
        }
        const int row = before[code >> 6] + (code & 63);
        a.inv_pos[p] = row;
        a.perm_src[row] = (int32_t)p;
    }
}

// Decode-sized batches (T <= 1024, S <= 256): rank, scan and the index
// outputs in one block of 1024 threads; wave w owns tokens [64w, 64w + 64).
constexpr int kSmallT = 1024, kSmallS = 256;

constexpr int kSmallE = 1024, kSmallNnz = 2048;

// KT > 0: top_k known at compile time (loads issued together, no branches);
// KT == 0: any top_k up to 16.
template <int KT>
__global__ __launch_bounds__(1024) void dispatch_small_kernel(DispatchArgs a) {
    constexpr int KMAX = KT > 0 ? KT : 16;
    const int K = KT > 0 ? KT : a.K;
    __shared__ unsigned long long masks[kSmallT / 64][kSmallS];
    __shared__ int base[kSmallT / 64][kSmallS];  // rows of earlier chunks, per slot
    __shared__ int offs[kSmallS + 1];
    __shared__ int scan[2][kSmallS];
    __shared__ int roff[kSmallE + 1];            // slot table staged in LDS
    __shared__ int rslot[kSmallNnz];
    const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
    const int C = (a.T + 63) / 64;
    const int t = tid;
    // this token's experts, loaded while the slot table is staged
    int ex[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) ex[k] = k < K && t < a.T ? a.topk_idx[(size_t)t * K + k] : -1;
    for (int i = tid; i < C * kSmallS; i += 1024) (&masks[0][0])[i] = 0ull;  // chunks in use
    for (int i = tid; i <= a.E; i += 1024) roff[i] = a.rep_off[i];
    const int nnz = a.rep_off[a.E];
    const bool table_in_lds = nnz >= 0 && nnz <= kSmallNnz;
    if (table_in_lds)
        for (int i = tid; i < nnz; i += 1024) rslot[i] = a.rep_slot[i];
    __syncthreads();
    const unsigned long long bit = 1ull << lane;
    int sls[KMAX];  // this thread's slots, kept for the final pass
    if (t < a.T) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) continue;  // (KT == 0) rounds past top_k
            const int e = ex[k];
            int sl = -1;
            if (e >= 0 && e < a.E) {
                const int lo = roff[e], n = roff[e + 1] - lo;
                if (n > 0) {
                    int r = 0;
                    if (n > 1)
                        r = (int)(splitmix64(a.seed ^ ((uint64_t)t * (uint64_t)K + (uint64_t)k)) %
                                  (uint64_t)n);
                    sl = table_in_lds ? rslot[lo + r] : a.rep_slot[lo + r];
                    if (sl < 0 || sl >= a.S) sl = -1;
                }
            }
            sls[k] = sl;
        }
        drop_repeated_slots<KMAX>(sls, K);
        int np = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) np += k < K && sls[k] >= 0;
        seed_tickets(a, t, np);
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < K && sls[k] >= 0) atomicOr(&masks[wave][sls[k]], bit);
    }
    __syncthreads();
    // per slot: exclusive scan over chunks, total
    int tot = 0;
    if (tid < a.S) {
        for (int c = 0; c < C; ++c) {
            base[c][tid] = tot;
            tot += __popcll(masks[c][tid]);
        }
        a.counts[tid] = tot;
    }
    // exclusive scan of totals over slots
    int cur = 0;
    if (tid < kSmallS) scan[0][tid] = tot;
    __syncthreads();
    for (int o = 1; o < kSmallS; o <<= 1) {
        if (tid < kSmallS) scan[cur ^ 1][tid] = scan[cur][tid] + (tid >= o ? scan[cur][tid - o] : 0);
        cur ^= 1;
        __syncthreads();
    }
    if (tid < a.S) {
        const int incl = scan[cur][tid];
        offs[tid] = incl - tot;
        a.offsets[tid] = incl - tot;
        if (tid == a.S - 1) {
            offs[a.S] = incl;
            a.offsets[a.S] = incl;
        }
    }
    __syncthreads();
    if (t < a.T)
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) continue;
            const size_t p = (size_t)t * K + k;
            const int sl = sls[k];
            if (sl < 0) {
                a.inv_pos[p] = -1;
                continue;
            }
            const int row = offs[sl] + base[wave][sl] + __popcll(masks[wave][sl] & (bit - 1ull));
            a.inv_pos[p] = row;
            a.perm_src[row] = (int32_t)p;
        }
}

__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    // |v| <= 448.  OCP E4M3: bias 7, 3 mantissa bits, subnormals below 2^-6.
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7fffffffu;
    if (a < 0x3c800000u) {  // |v| < 2^-6: multiples of 2^-9, RNE
        const float q = __uint_as_float(a) * 512.0f;
        return sign | (uint32_t)__builtin_rintf(q);
    }
    // keep exponent and top 3 mantissa bits, round the low 20 bits to nearest even
    uint32_t q = a >> 20;
    const uint32_t rem = a & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1u;
    return sign | (q - ((127u - 7u) << 3));
}

// Row copy for rows placed already (inv_pos written), one wave per pair:
// the fallback for rows longer than dispatch_rows_kernel holds.
template <typename T, int XM>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(DispatchArgs a) {
    const size_t p = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= (size_t)a.T * a.K) return;
    const int lane = lane_id();
    const int t = (int)(p / a.K);
    const int row = __builtin_amdgcn_readfirstlane(a.inv_pos[p]);
    if (row < 0) return;
    constexpr int EL = Frag<T>::kElems;
    const T *src = reinterpret_cast<const T *>(a.h) + (size_t)t * a.H;
    if (XM != DT_FP8) {
        T *dst = reinterpret_cast<T *>(a.x_perm) + (size_t)row * a.H;
        for (int i = lane * EL; i < a.H; i += 64 * EL)
            *reinterpret_cast<typename Frag<T>::vec *>(dst + i) = load16(src + i);
        return;
    }
    // FP8: per-row amax -> scale, then codes
    float amax = 0.0f;
    for (int i = lane * EL; i < a.H; i += 64 * EL) {
        const typename Frag<T>::vec v = load16(src + i);
#pragma unroll
        for (int j = 0; j < EL; ++j) amax = fmaxf(amax, fabsf((float)v[j]));
    }
    amax = wave_max(amax);
    uint8_t *dst = reinterpret_cast<uint8_t *>(a.x_perm) + (size_t)row * a.H;
    if (amax == 0.0f) {
        for (int i = lane * EL; i < a.H; i += 64 * EL)
            *reinterpret_cast<u32x2 *>(dst + i) = u32x2{0u, 0u};
        if (lane == 0) a.x_scale[row] = 0.0f;
        return;
    }
    const float inv = __fdiv_rn(448.0f, amax);
    if (lane == 0) a.x_scale[row] = __fdiv_rn(amax, 448.0f);
    for (int i = lane * EL; i < a.H; i += 64 * EL) {
        const typename Frag<T>::vec v = load16(src + i);
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < EL; ++j) {
            float q = __fmul_rn((float)v[j], inv);
            q = fminf(fmaxf(q, -448.0f), 448.0f);
            w[j >> 2] |= e4m3_rne(q) << (8 * (j & 3));
        }
        *reinterpret_cast<u32x2 *>(dst + i) = u32x2{w[0], w[1]};
    }
}

// One block of 256 threads per token: the token's hidden row is read once
// into registers (every load issued before the first use) and written --
// copied, or quantised once to E4M3 codes with one scale -- to each local
// row the token was dispatched to.  Tokens with no local pair read nothing.
// H <= 256 * EL * kRowSteps.
constexpr int kRowSteps = 4;

template <typename T, int XM>
__global__ __launch_bounds__(256) void dispatch_rows_kernel(DispatchArgs a) {
    __shared__ float wmax[4];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    // every wave reads the token's K row indices: the same ballot in all 4
    const int myrow = lane < a.K ? a.inv_pos[(size_t)t * a.K + lane] : -1;
    uint64_t todo = __ballot(myrow >= 0);
    if (!todo) return;  // block-uniform
    constexpr int EL = Frag<T>::kElems;
    typedef typename Frag<T>::vec V;
    const T *src = reinterpret_cast<const T *>(a.h) + (size_t)t * a.H;
    V v[kRowSteps];
#pragma unroll
    for (int i = 0; i < kRowSteps; ++i) {
        const int c = (i * 256 + tid) * EL;
        if (c < a.H) v[i] = load16(src + c);
    }
    if (XM != DT_FP8) {
        while (todo) {
            const int k = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int row = __builtin_amdgcn_readlane(myrow, k);
            T *dst = reinterpret_cast<T *>(a.x_perm) + (size_t)row * a.H;
#pragma unroll
            for (int i = 0; i < kRowSteps; ++i) {
                const int c = (i * 256 + tid) * EL;
                if (c < a.H) *reinterpret_cast<V *>(dst + c) = v[i];
            }
        }
        return;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowSteps; ++i)
        if ((i * 256 + tid) * EL < a.H)
#pragma unroll
            for (int j = 0; j < EL; ++j) amax = fmaxf(amax, fabsf((float)v[i][j]));
    amax = wave_max(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    // amax == 0: all codes and the scale are 0
    const float inv = amax == 0.0f ? 0.0f : __fdiv_rn(448.0f, amax);
    const float scale = amax == 0.0f ? 0.0f : __fdiv_rn(amax, 448.0f);
    u32x2 codes[kRowSteps];
#pragma unroll
    for (int i = 0; i < kRowSteps; ++i) {
        uint32_t w[2] = {0u, 0u};
        if (amax != 0.0f && (i * 256 + tid) * EL < a.H)
#pragma unroll
            for (int j = 0; j < EL; ++j) {
                float q = __fmul_rn((float)v[i][j], inv);
                q = fminf(fmaxf(q, -448.0f), 448.0f);
                w[j >> 2] |= e4m3_rne(q) << (8 * (j & 3));
            }
        codes[i] = u32x2{w[0], w[1]};
    }
    while (todo) {
        const int k = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int row = __builtin_amdgcn_readlane(myrow, k);
        uint8_t *dst = reinterpret_cast<uint8_t *>(a.x_perm) + (size_t)row * a.H;
#pragma unroll
        for (int i = 0; i < kRowSteps; ++i) {
            const int c = (i * 256 + tid) * EL;
            if (c < a.H) *reinterpret_cast<u32x2 *>(dst + c) = codes[i];
        }
        if (tid == 0) a.x_scale[row] = scale;
    }
}

}  // namespace

size_t dispatch_scratch_bytes(int T, int K, int S) {
    const size_t C = (size_t)(T + 63) / 64;
    size_t a = ((size_t)T * K * 4 + 255) & ~(size_t)255;
    a += ((C * (size_t)S * 4) + 255) & ~(size_t)255;
    return a;
}

// Row copies once inv_pos is written (x_perm != NULL).
hipError_t launch_rows(const DispatchArgs &a, hipStream_t s) {
    const int EL = a.dtype == DT_F32 ? 4 : 8;
    if (a.H <= 256 * EL * kRowSteps) {
        dim3 grid((unsigned)a.T);
        if (a.dtype == DT_F32)
            hipLaunchKernelGGL((dispatch_rows_kernel<float, DT_F32>), grid, dim3(256), 0, s, a);
        else if (a.x_dtype == DT_FP8)
            hipLaunchKernelGGL((dispatch_rows_kernel<f16, DT_FP8>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((dispatch_rows_kernel<f16, DT_F16>), grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const size_t pairs = (size_t)a.T * a.K;
    dim3 grid((unsigned)((pairs + 3) / 4));
    if (a.dtype == DT_F32)
        hipLaunchKernelGGL((dispatch_scatter_kernel<float, DT_F32>), grid, dim3(256), 0, s, a);
    else if (a.x_dtype == DT_FP8)
        hipLaunchKernelGGL((dispatch_scatter_kernel<f16, DT_FP8>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((dispatch_scatter_kernel<f16, DT_F16>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s) {
    if (a.T < 0) return hipErrorInvalidValue;
    const int C = (a.T + 63) / 64;
    hipError_t e;
    if (a.T > 0 && a.T <= kSmallT && a.S <= kSmallS && a.E <= kSmallE) {
        if (a.K == 8)
            hipLaunchKernelGGL(dispatch_small_kernel<8>, dim3(1), dim3(1024), 0, s, a);
        else if (a.K == 2)
            hipLaunchKernelGGL(dispatch_small_kernel<2>, dim3(1), dim3(1024), 0, s, a);
        else
            hipLaunchKernelGGL(dispatch_small_kernel<0>, dim3(1), dim3(1024), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (!a.x_perm) return hipSuccess;  // rows are gathered by the GEMM instead
        return launch_rows(a, s);
    }
    if (C > 0) {
        hipLaunchKernelGGL(dispatch_rank_kernel, dim3((C + 3) / 4), dim3(256),
                           (size_t)4 * a.S * sizeof(unsigned long long), s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (C > 0 && a.S <= kPlaceMaxS && (long)C * a.S <= kPlaceMaxTable) {
        hipLaunchKernelGGL(dispatch_place_kernel, dim3(C), dim3(256), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess || !a.x_perm) return e;
        return launch_rows(a, s);
    }
    // with T = 0 the scan alone writes all-zero counts and offsets
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.T == 0) return hipSuccess;
    const size_t pairs = (size_t)a.T * a.K;
    hipLaunchKernelGGL(dispatch_index_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                       s, a);
    e = hipGetLastError();
    if (e != hipSuccess || !a.x_perm) return e;
    return launch_rows(a, s);
}

}  // namespace moe
