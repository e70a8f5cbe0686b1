// gemm_tiled.hip -- grouped LDS-tiled MFMA GEMM for large row counts (prefill).
//
// Same contract as the weight-stream kernel (router logits, SwiGLU gate/up,
// down projection; Steps 1 and 3 of the expert-parallelism blog page, section
// 2.2), for groups that hold hundreds of rows.  There every weight tile is
// reused by many rows, so the work is bound by the matrix cores (the PPIO
// essay: prefill is compute-bound) and both operands are staged through LDS.
//
//   out[r][n] = epilogue( sum_k W[g][n][k] * x[r][k] )   rows r of group g
//
// Tiles: 256 x rows (expert GEMMs) or 128 (router) by 256 weight rows (128
// features x gate and up for SwiGLU, 256 features otherwise), BK = 64.
// 512 threads = 8 waves (2 per SIMD) in a 2 x 4 arrangement; each wave owns
// TBM/2 rows x 64 weight rows as tiles of v_mfma_f32_16x16x32_f16.
// Operands go from global memory straight into LDS (buffer/global loads with
// the lds modifier: no register staging), two stages for 256-row tiles and
// three for 128-row ones, one barrier per K step, XOR-swizzled LDS rows (see
// swz()).  Expert weights in the fragment layout (frag_offset) are staged
// fragment by fragment: one wave load is one contiguous 1 KB fragment and
// lands in LDS in the order the MFMA reads it (lane l's 16 bytes at 16 l),
// so those reads need no swizzle.
//
// The grid is persistent (all resident workgroup slots): see tiled_gemm_kernel;
// a workgroup's items share one pipeline where rows are not gathered (see
// run_items_dma).
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int WNW = 4;               // waves along the weight rows (2 x 4 waves)
constexpr int WR = 64 * WNW;         // weight rows per tile (gate + up halves for SwiGLU)
constexpr int BK = 64;               // reduction per pipeline step
constexpr int PITCH = BK;            // halves per LDS row (128 B, XOR-swizzled chunks)
constexpr int kThreads = 128 * WNW;  // 2 x WNW waves
constexpr int kExpertRows = 256;     // x rows per tile of the expert GEMMs
constexpr int kMaxDevices = 64;

// LDS offset (halves) of 16-byte chunk c of row r: the chunk index is XORed
// with r % 8, so the 16 rows one MFMA fragment read touches spread over all
// banks (a 16-byte row pad still leaves 2-way conflicts on gfx950, as
// measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz(int r, int c) { return r * PITCH + ((c ^ (r & 7)) << 3); }

// One work item: x rows [rs, rs + tile rows) of group g x features
// [n0, n0 + WR/NM), K slice kz (router logits only).  Everything a load or
// the epilogue needs.
template <int NM>
struct Item {
    int rs, r1, n0, kz, k0;                // rows, features, K slice, K offset
    const f16 *xb, *wb[NM];                // this tile's x rows and weight rows
    int xbytes, wbytes;                    // their byte ranges
};

template <int NM, int EPI, int TBM>
__device__ __forceinline__ Item<NM> make_item(const StreamArgs &a, int g, int mt, int nt, int kz,
                                              int nk) {
    constexpr int FN = WR / NM;  // features per tile
    // wave-uniform by construction; readfirstlane keeps them (and the
    // ranges formed from them) in scalar registers
    g = __builtin_amdgcn_readfirstlane(g);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    kz = __builtin_amdgcn_readfirstlane(kz);
    int r0, r1;
    if (a.offsets) {
        r0 = a.offsets[g];
        r1 = a.offsets[g + 1];
    } else {
        r0 = g * a.rows_per_group;
        r1 = r0 + a.rows_per_group;
    }
    r0 = __builtin_amdgcn_readfirstlane(r0);
    r1 = __builtin_amdgcn_readfirstlane(r1);
    Item<NM> it;
    it.rs = r0 + mt * TBM;
    it.r1 = r1;
    it.n0 = nt * FN;
    it.kz = kz;
    it.k0 = EPI == 2 ? kz * nk * BK : 0;
    const int K = a.K;
    // Loads go through buffer descriptors over [xb, xb + xbytes) and
    // [wb, wb + wbytes): rows past the tile's valid rows fall outside the
    // range and load zeros, so no clamping is needed.
    const int rows_valid = (r1 - it.rs) < TBM ? (r1 - it.rs) : TBM;
    const int xrow0 = a.x_broadcast ? it.rs - r0 : it.rs;
    it.xb = reinterpret_cast<const f16 *>(a.x) + (size_t)xrow0 * K;
    it.xbytes = rows_valid * K * 2;
    const int ncols = (a.N - it.n0) < FN ? (a.N - it.n0) : FN;
    it.wbytes = ncols * K * 2;
#pragma unroll
    for (int m = 0; m < NM; ++m)
        it.wb[m] = reinterpret_cast<const f16 *>(m == 0 ? a.w0 : a.w1) +
                   (size_t)g * a.w_group_stride + (size_t)it.n0 * K;
    return it;
}

// The items of one workgroup, in order: item j is seq.first + j*seq.step
// (< seq.end), decoded to (group, row tile, feature tile, K slice).
struct ItemSeq {
    int first, step, end;
    bool chunked;  // (group, feature tile, row tile) order, else (row tile, feature tile, slice)
};

__device__ __forceinline__ void decode_item(const int *tstart, int n_groups, int n_ntiles, int ks,
                                            bool chunked, int item, int &g, int &mt, int &nt,
                                            int &kz) {
    int lo = 0, hi = n_groups - 1;
    if (chunked) {
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tstart[mid] * n_ntiles <= item)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int tg = tstart[lo + 1] - tstart[lo];  // row tiles of group lo
        const int local = item - tstart[lo] * n_ntiles;
        g = lo;
        mt = local % tg;
        nt = local / tg;
        kz = 0;
    } else {
        kz = item % ks;
        const int tile = item / ks / n_ntiles;
        nt = (item / ks) % n_ntiles;
        // group holding this row tile: last g with tstart[g] <= tile
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tstart[mid] <= tile)
                lo = mid;
            else
                hi = mid - 1;
        }
        g = lo;
        mt = tile - tstart[g];
    }
}

// Tile geometry of the direct-to-LDS pipeline: K steps of BK, two LDS
// stages of 64 KB for 256-row tiles, three of 48 KB for 128-row ones.
template <int TBM>
constexpr int n_stages() {
    return TBM == 256 ? 2 : 3;
}

// ---- direct global -> LDS staging (gfx950 buffer/global loads with the lds
// modifier).  Lane l of one such load writes its 16 bytes to LDS byte
// M0 + 16 l, so one wave instruction fills 1 KB = 8 rows of 128 B; the XOR
// swizzle of swz() is applied on the global side (lane l of a block of 8
// rows fetches global chunk (l % 8) ^ (l / 8) of row l / 8).  The loads are
// issued from inline asm so that the compiler does not order every LDS read
// behind every load in flight (it cannot tell the stages apart); completion
// is waited for explicitly (vmcnt, in issue order) before the barrier that
// publishes a stage.  M0 is written here and used by nothing else in these
// kernels.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// Raw buffer descriptor (base, byte range; stride 0) held in scalar registers.
__device__ __forceinline__ u32x4 srd(const void *base, int bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
    r[3] = 0x00020000u;
    return r;
}
__device__ __forceinline__ void dma_buf16(u32x4 r, uint32_t m0, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0),
                 "v"(voff), "s"(r), "s"(soff)
                 : "memory");
}
__device__ __forceinline__ void dma_glb16(const void *p, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(p)
                 : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The items of one workgroup with direct-to-LDS staging.  Tiles of TBM x
// rows (128 or 256) by 256 weight rows; 8 waves in 2 (rows) x 4 (weight
// rows), wave (wm, wn) owning TBM/2 rows x 64 weight rows.  128-row tiles use
// three LDS stages (the loads of step k+2 issued at the start of step k),
// 256-row tiles two (step k+1's loads issued at the start of step k; a step
// is twice as long), so a load has about 2048 MFMA cycles to land either way.
// Wave w stages x rows w*TBM/8..+TBM/8 and weight rows w*32..+32 of every
// step.  A wave whose rows all lie past the group's end (the last, partly
// filled row tile of a group) skips its fragment reads and MFMAs.  Items
// chain (the steps past an item's end load the next item's first ones)
// unless x rows are gathered.
template <int TBM, int NM, int EPI, bool GATHER, bool FR>
__device__ __forceinline__ void run_items_dma(const StreamArgs &a, f16 *As, f16 *Bs,
                                              const int *tstart, int n_groups, int n_ntiles,
                                              int ks, const ItemSeq seq) {
    constexpr int FN = WR / NM;
    constexpr int NJ = 4 / NM;
    constexpr int WMR = TBM / 2;           // rows per wave
    constexpr int MI = WMR / 16;           // 16-row subtiles per wave
    constexpr int NSTG = n_stages<TBM>();
    constexpr int LOOK = NSTG - 1;         // steps loaded ahead
    constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
    constexpr int RPI = 64 / CPR;          // rows one wave load fills (1 KB)
    constexpr int XW = TBM / 8;            // x rows one wave stages
    constexpr int XL = XW / RPI;           // wave loads of x rows per step
    constexpr int WL = 32 / RPI;           // of weight rows (32 per wave)
    static_assert(TBM == 128 || TBM == 256, "tile height");
    const int K = a.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WNW, wn = wave % WNW;
    const int lr = lane & 15, lg = lane >> 4;
    const int nk = EPI == 2 ? K / BK / a.ksplit : K / BK;
    const bool chain = !GATHER;

    // this lane's source row within the block one wave load fills and its
    // (swizzled) chunk: the row's swizzle key depends only on its offset in
    // the block
    const int rsub = lane / CPR, gch = (lane % CPR) ^ (rsub & 7);
    int xoff[XL], woff[WL];
#pragma unroll
    for (int i = 0; i < XL; ++i) xoff[i] = (wave * XW + i * RPI + rsub) * K * 2 + gch * 16;
    const int wmat = (wave * 32) / FN;  // the weight matrix this wave stages
    // fragment layout: load i is fragment (16-row group wr0/16 + i/2, 64-byte
    // K chunk i%2 of the step); LDS holds a stage's fragments in (row group,
    // chunk) order, 2 KB per row group.  The step's K offset kb (bytes of a
    // row-major row) is 16 kb bytes into the fragments.
    static_assert(!FR || WL == 4, "a wave stages two row groups x two K chunks");
    const int wr0 = (wave * 32) % FN;  // first row this wave stages, in its matrix
#pragma unroll
    for (int i = 0; i < WL; ++i)
        woff[i] = FR ? ((wr0 / 16 + i / 2) * (K / 32) + i % 2) * 1024 + lane * 16
                     : ((wave * 32 + i * RPI + rsub) % FN) * K * 2 + gch * 16;
    constexpr int ASTAGE = TBM * BK * 2, BSTAGE = WR * BK * 2;  // bytes
    const uint32_t a_m0 = lds_addr(As) + wave * XW * BK * 2;
    const uint32_t b_m0 = lds_addr(Bs) + wave * 32 * BK * 2;

    // gathered rows: this lane's source row of each of its x loads
    const f16 *xg[XL];
    auto set_gather = [&](const Item<NM> &it) {
        if (GATHER) {
#pragma unroll
            for (int i = 0; i < XL; ++i) {
                int r = it.rs + wave * XW + i * RPI + rsub;
                if (r > it.r1 - 1) r = it.r1 - 1;
                xg[i] = reinterpret_cast<const f16 *>(a.x) +
                        (size_t)(a.gather[r] / a.gather_div) * K + gch * 8;
            }
        }
    };
    // stage K step s of the chain into LDS stage st (steps past the current
    // item's end: the next item's, or a harmless re-load of the last step)
    auto stage = [&](const Item<NM> &cur, const Item<NM> &nxt, bool has_nxt, int s, int st) {
        const bool to_nxt = s >= nk && has_nxt;
        const int sk = s < nk ? s : (to_nxt ? s - nk : nk - 1);
        const int kb = __builtin_amdgcn_readfirstlane(((to_nxt ? nxt.k0 : cur.k0) + sk * BK) * 2);
        if (GATHER) {
#pragma unroll
            for (int i = 0; i < XL; ++i)
                dma_glb16(xg[i] + kb / 2, a_m0 + st * ASTAGE + i * 1024);
        } else {
            const u32x4 xr = to_nxt ? srd(nxt.xb, nxt.xbytes) : srd(cur.xb, cur.xbytes);
#pragma unroll
            for (int i = 0; i < XL; ++i) dma_buf16(xr, a_m0 + st * ASTAGE + i * 1024, xoff[i], kb);
        }
        // (a select, not an index: a run-time index would put the items in
        // scratch memory)
        const f16 *wb0 = to_nxt ? nxt.wb[0] : cur.wb[0];
        const f16 *wb1 = to_nxt ? nxt.wb[NM - 1] : cur.wb[NM - 1];
        const u32x4 wr = srd(wmat == 0 ? wb0 : wb1, to_nxt ? nxt.wbytes : cur.wbytes);
#pragma unroll
        for (int i = 0; i < WL; ++i)
            dma_buf16(wr, b_m0 + st * BSTAGE + i * 1024, woff[i], FR ? kb * 16 : kb);
    };

    // Fragment reads: the weight fragments first, then the row fragments in
    // the order the MFMAs consume them (row subtile outer), so a wave's first
    // MFMA waits for NM*NJ + 1 reads and each later row fragment feeds NM*NJ
    // MFMAs.
    f16x8 af0[MI], bf0[NM][NJ], af1[MI], bf1[NM][NJ];
    // (scheduling barriers keep the compiler from moving the row reads ahead)
    auto fread = [&](f16x8 *af, f16x8 (*bf)[NJ], int st, int kq) {
        const f16 *A = As + st * TBM * BK;
        const f16 *B = Bs + st * WR * BK;
        const int ch = kq + lg;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int wrow = m * FN + wn * (FN / WNW) + j * 16;  // fragment's first row
                bf[m][j] = *reinterpret_cast<const f16x8 *>(
                    FR ? B + ((wrow / 16) * 2 + kq / 4) * 512 + lane * 8 : B + swz(wrow + lr, ch));
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MI; ++i)
            af[i] = *reinterpret_cast<const f16x8 *>(A + swz(wm * WMR + i * 16 + lr, ch));
        __builtin_amdgcn_sched_barrier(0);
    };
    f32x4 acc[NM][MI][NJ];
    // MFMAs of row subtiles [i0, i1)
    auto mm = [&](const f16x8 *af, f16x8 (*bf)[NJ], int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[m][i][j] = mfma16(af[i], bf[m][j], acc[m][i][j]);
    };
    auto next_stage = [](int st) { return st + 1 == NSTG ? 0 : st + 1; };
    auto zero_acc = [&]() {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // acc[m][i][j]: x row wm*WMR + i*16 + 4*lg + q (q = 0..3), feature
    // n0 + wn*FN/4 + j*16 + lr.
    auto epilogue = [&](const Item<NM> &it) {
        if constexpr (EPI == 2) {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = it.rs + wm * WMR + i * 16 + 4 * lg + q;
                    if (r >= it.r1) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int f = it.n0 + wn * (FN / WNW) + j * 16 + lr;
                        if (f >= a.N) continue;
                        reinterpret_cast<float *>(a.out)[(size_t)it.kz * a.split_stride +
                                                         (size_t)r * a.out_ld + f] =
                            acc[0][i][j][q];
                    }
                }
            }
        } else {
            // fp16 results two features per store: lanes l and l^1 hold the
            // same 4 rows at adjacent features; they swap two values (DPP
            // quad_perm [1,0,3,2]) so the even lane writes rows q = 0, 1 and
            // the odd lane rows 2, 3, each as one 4-byte store
            const bool odd = lr & 1;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    uint32_t h[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float v = EPI == 1
                                            ? siluf_(acc[0][i][j][q]) * acc[NM - 1][i][j][q]
                                            : acc[0][i][j][q];
                        h[q] = (uint32_t)__builtin_bit_cast(uint16_t, to_f16(v));
                    }
                    const uint32_t s0 = odd ? h[0] : h[2], s1 = odd ? h[1] : h[3];
                    const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xf, 0xf, false);
                    const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xf, 0xf, false);
                    // even lane: rows q0, q1 = (own, partner); odd: rows q2, q3 = (partner, own)
                    const uint32_t w0 = odd ? (r0 | (h[2] << 16)) : (h[0] | (r0 << 16));
                    const uint32_t w1 = odd ? (r1 | (h[3] << 16)) : (h[1] | (r1 << 16));
                    const int f = it.n0 + wn * (FN / WNW) + j * 16 + (lr & ~1);
                    const int rb = it.rs + wm * WMR + i * 16 + 4 * lg + (odd ? 2 : 0);
                    if (f < a.N) {
                        uint32_t *o0 = reinterpret_cast<uint32_t *>(reinterpret_cast<f16 *>(a.out) +
                                                                    (size_t)rb * a.out_ld + f);
                        uint32_t *o1 = reinterpret_cast<uint32_t *>(reinterpret_cast<f16 *>(a.out) +
                                                                    (size_t)(rb + 1) * a.out_ld + f);
                        if (rb < it.r1) *o0 = w0;
                        if (rb + 1 < it.r1) *o1 = w1;
                    }
                }
            }
        }
    };

    if (seq.first >= seq.end) return;
    int g, mt, nt, kz;
    decode_item(tstart, n_groups, n_ntiles, ks, seq.chunked, seq.first, g, mt, nt, kz);

    Item<NM> cur = make_item<NM, EPI, TBM>(a, g, mt, nt, kz, nk);
    Item<NM> nxt = cur;
    int inext = seq.first + seq.step;
    bool primed = false;
    int sc = 0;  // stage of step kt
    for (;;) {
        const bool has_nxt = chain && inext < seq.end;
        if (has_nxt) {
            decode_item(tstart, n_groups, n_ntiles, ks, seq.chunked, inext, g, mt, nt, kz);
            nxt = make_item<NM, EPI, TBM>(a, g, mt, nt, kz, nk);
        }
        if (!primed) {
            set_gather(cur);
            int st = sc;
#pragma unroll
            for (int j = 0; j < LOOK; ++j) {
                stage(cur, nxt, false, j, st);
                st = next_stage(st);
            }
        }
        // wave-uniform: does this wave own any row of the tile?
        const bool live = cur.rs + wm * WMR < cur.r1;
        zero_acc();
        for (int kt = 0; kt < nk; ++kt) {
            // this wave's loads of step kt are in; the barrier publishes every
            // wave's and retires the reads of step kt-1's stage, which the
            // loads of step kt+LOOK then refill
            wait_vm<(LOOK - 1) * (XL + WL)>();
            __syncthreads();
            const int sl = sc + LOOK < NSTG ? sc + LOOK : sc + LOOK - NSTG;
            stage(cur, nxt, has_nxt, kt + LOOK, sl);
            if (live) {
                // the first K half's fragments, half of its MFMAs, the second
                // half's fragments (landing during the rest), the remaining
                // MFMAs: at most 2*(MI + NM*NJ) reads in flight and no MFMA
                // waits for more than the first NM*NJ + 1 of them (the LDS
                // counter holds 15)
                fread(af0, bf0, sc, 0);
                mm(af0, bf0, 0, MI / 2);
                fread(af1, bf1, sc, 4);
                mm(af0, bf0, MI / 2, MI);
                mm(af1, bf1, 0, MI);
                __builtin_amdgcn_sched_barrier(0);
            }
            sc = next_stage(sc);
        }

        if (live) epilogue(cur);
        if (!has_nxt && inext >= seq.end) break;
        primed = has_nxt;
        if (!has_nxt) {
            // restart: let the dummy loads land and every wave finish reading
            // before the stages are refilled
            wait_vm<0>();
            __syncthreads();
            decode_item(tstart, n_groups, n_ntiles, ks, seq.chunked, inext, g, mt, nt, kz);
            nxt = make_item<NM, EPI, TBM>(a, g, mt, nt, kz, nk);
            sc = 0;
        }
        cur = nxt;
        inext += seq.step;
    }
    wait_vm<0>();
}

// ---- The combine in the down projection (comb.out set) ----
// Steps 4-5 of the EP blog page (section 2.2) in this launch's tail: the page
// lets the combine run alongside the last expert computations (section 2.3),
// and the large-EP article (三.2) fuses the gather and the scatter around the
// grouped GEMM.  Result, per token t and feature i:
//   out[t][i] = sum over t's local pairs k (k order) of topk_w[t][k] * y[inv_pos[t][k]][i]
//               + shared_gate[t] * sum_j shared_y[j][t][i]
// with the combine kernel's arithmetic (fp32 fma from 0 in that order, one
// rounding), so the bits equal the separate combine's.
//
// Dispatch set one ticket per (token, 256-feature tile) to the token's local
// pair count.  A workgroup that has finished its items makes its y rows
// visible at agent scope (release fence), takes the ticket of every (row,
// feature tile) it wrote (atomic decrement), and sums the (token, tile)s
// whose ticket it took to zero -- it wrote the last of their rows -- after
// an acquire fence, reading the other pairs' rows from memory.  No workgroup
// waits for another, so nothing depends on workgroups being co-resident.
// Tokens with no local pair (their experts live on other ranks) get zeros,
// or the shared term alone, from workgroup t mod grid.
constexpr int kCombSub = kThreads;  // entries summed per pass (one pair list per thread)
constexpr int kCombCap = 4096;      // list room: under kCombSub pending + one batch's 4 x kThreads
constexpr int kCombMaxK = 16;       // top-K limit of the shape check
static_assert(kCombCap >= kCombSub - 1 + 4 * kThreads, "list room");
constexpr size_t kCombLds =
    (size_t)kCombCap * 4 + (size_t)kCombSub * kCombMaxK * 8 + (size_t)kCombSub * 3 * 4;

__device__ __forceinline__ f16x8 ldg16(const f16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

template <int TBM>
__device__ void comb_tail(const StreamArgs &a, const ItemSeq &seq, const int *tstart, int n_groups,
                          int n_ntiles, f16 *lds) {
    static_assert(TBM == 256 && kThreads == 512, "one row of two items per thread");
    const CombineArgs &c = a.comb;
    const int tid = threadIdx.x;
    const int K = c.K, H = a.N, T = c.T, nft = n_ntiles;
    const bool sh = c.shared_y && c.n_shared > 0;
    const f16 *y = reinterpret_cast<const f16 *>(a.out);
    const f16 *shy = reinterpret_cast<const f16 *>(c.shared_y);
    f16 *out = reinterpret_cast<f16 *>(c.out);
    int *list = reinterpret_cast<int *>(lds);          // [kCombCap] ticket indices t*nft + f
    int *prow = list + kCombCap;                       // [kCombSub][kCombMaxK] local rows, k order
    float *pw = reinterpret_cast<float *>(prow + kCombSub * kCombMaxK);  // their weights
    int *pn = reinterpret_cast<int *>(pw + kCombSub * kCombMaxK);       // local pair count
    int *pe = pn + kCombSub;                                            // ticket index
    float *pgs = reinterpret_cast<float *>(pe + kCombSub);              // shared gate
    __shared__ int nlist;

    // 8 features from i of token t: the pairs' rows (np of them, from LDS
    // row-lists at rl / wl), then the shared term; stored to out.
    // (4 units per thread, their loads in flight together)
    auto sum_units = [&](int units, auto unit_of) {
        for (int u0 = tid; u0 < units; u0 += 4 * kThreads) {
            int t[4], i[4], np[4], base[4];
            float gs[4];
            int maxnp = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                np[q] = -1;
                const int u = u0 + q * kThreads;
                if (u < units) unit_of(u, t[q], i[q], np[q], base[q], gs[q]);
                maxnp = np[q] > maxnp ? np[q] : maxnp;
            }
            float acc[4][8];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[q][j] = 0.f;
            for (int k0 = 0; k0 < maxnp; k0 += 4) {
                f16x8 v[4][4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        if (k0 + kk < np[q])
                            v[q][kk] = ldg16(y + (size_t)prow[base[q] + k0 + kk] * H + i[q]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        if (k0 + kk < np[q]) {
                            const float g = pw[base[q] + k0 + kk];
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                acc[q][j] = __builtin_fmaf(g, (float)v[q][kk][j], acc[q][j]);
                        }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (np[q] < 0) continue;
                if (sh) {
                    float sv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                    for (int s = 0; s < c.n_shared; ++s) {
                        const f16x8 w = ldg16(shy + ((size_t)s * T + t[q]) * H + i[q]);
#pragma unroll
                        for (int j = 0; j < 8; ++j) sv[j] += (float)w[j];
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[q][j] = __builtin_fmaf(gs[q], sv[j], acc[q][j]);
                }
                f32x8 a8;
#pragma unroll
                for (int j = 0; j < 8; ++j) a8[j] = acc[q][j];
                *reinterpret_cast<f16x8 *>(out + (size_t)t[q] * H + i[q]) = to_f16x8_of_f32(a8);
            }
        }
    };

    // sum the n (token, tile) entries of the list
    auto flush = [&](int n) {
        // see the rows the other producers released before their decrements
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        for (int b = 0; b < n; b += kCombSub) {
            const int m = n - b < kCombSub ? n - b : kCombSub;
            if (tid < m) {
                const int e = list[b + tid];
                const int t = e / nft;
                // all K loads in flight together, then compacted in k order
                int r[kCombMaxK];
                float w[kCombMaxK];
#pragma unroll
                for (int k = 0; k < kCombMaxK; ++k) {
                    r[k] = k < K ? c.inv_pos[(size_t)t * K + k] : -1;
                    w[k] = k < K ? c.topk_w[(size_t)t * K + k] : 0.f;
                }
                int np = 0;
#pragma unroll
                for (int k = 0; k < kCombMaxK; ++k)
                    if (r[k] >= 0) {
                        prow[tid * kCombMaxK + np] = r[k];
                        pw[tid * kCombMaxK + np] = w[k];
                        ++np;
                    }
                pn[tid] = np;
                pe[tid] = e;
                pgs[tid] = sh ? c.shared_gate[t] : 0.f;
            }
            __syncthreads();
            // units: (entry, 8-feature chunk), 32 chunks per 256-feature tile
            sum_units(m * (WR / 8), [&](int u, int &t, int &i, int &np, int &base, float &gs) {
                const int ent = u / (WR / 8);
                const int e = pe[ent];
                t = e / nft;
                i = (e - t * nft) * WR + (u % (WR / 8)) * 8;
                if (i >= H) return;  // past the last, narrower tile
                np = pn[ent];
                base = ent * kCombMaxK;
                gs = pgs[ent];
            });
            __syncthreads();
        }
    };

    // every wave's y stores have completed (run_items_dma waited for them)
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (tid == 0) nlist = 0;
    __syncthreads();
    const int nitems = seq.first < seq.end ? (seq.end - seq.first + seq.step - 1) / seq.step : 0;
    // items in batches of 8: thread tid takes row tid % 256 of items 2q + tid / 256
    for (int b0 = 0; b0 < nitems; b0 += 8) {
        int row[4], ft[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            row[q] = -1;
            ft[q] = 0;
            const int j = b0 + 2 * q + (tid >> 8);
            if (j < nitems) {
                int g, mt, nt, kz;
                decode_item(tstart, n_groups, n_ntiles, 1, seq.chunked, seq.first + j * seq.step, g,
                            mt, nt, kz);
                const int r0 = a.offsets ? a.offsets[g] : g * a.rows_per_group;
                const int r1 = a.offsets ? a.offsets[g + 1] : r0 + a.rows_per_group;
                const int r = r0 + mt * TBM + (tid & 255);
                if (r < r1) {
                    row[q] = r;
                    ft[q] = nt;
                }
            }
        }
        int pair[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) pair[q] = row[q] >= 0 ? c.perm_src[row[q]] : -1;
        int tk[4], left[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            left[q] = -1;
            tk[q] = pair[q] >= 0 ? (pair[q] / K) * nft + ft[q] : -1;
            if (tk[q] >= 0)
                left[q] = __hip_atomic_fetch_add(c.tickets + tk[q], -1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (tk[q] >= 0 && left[q] == 1) list[atomicAdd(&nlist, 1)] = tk[q];
        __syncthreads();
        const int n = nlist;
        // every thread has its n before any appends again: all take the
        // same branch (flush holds barriers)
        __syncthreads();
        if (n >= kCombSub) {  // a full pass is pending: sum it now
            flush(n);
            if (tid == 0) nlist = 0;
            __syncthreads();
        }
    }
    __syncthreads();
    if (nlist > 0) flush(nlist);

    // tokens without a local pair: zeros, or the shared term alone
    const int G = gridDim.x;
    for (int t0 = blockIdx.x; t0 < T; t0 += G * kThreads) {
        __syncthreads();
        if (tid == 0) nlist = 0;
        __syncthreads();
        const int t = t0 + tid * G;
        if (t < T) {
            bool any = false;
#pragma unroll
            for (int k = 0; k < kCombMaxK; ++k)
                if (k < K) any |= c.inv_pos[(size_t)t * K + k] >= 0;
            if (!any) {
                const int at = atomicAdd(&nlist, 1);
                list[at] = t;
                pgs[at] = sh ? c.shared_gate[t] : 0.f;
            }
        }
        __syncthreads();
        const int nz = nlist;
        sum_units(nz * (H / 8), [&](int u, int &t, int &i, int &np, int &base, float &gs) {
            const int ent = u / (H / 8);
            t = list[ent];
            i = (u % (H / 8)) * 8;
            np = 0;
            base = 0;
            gs = pgs[ent];
        });
    }
}

constexpr int kMaxGroups = 1024;

// Persistent: a fixed grid walks the real tiles.  Each workgroup first builds
// the prefix of row tiles per group from the device-side offsets (group
// sizes are only known on the device), then runs its share of the items.
// Expert GEMMs (grid a multiple of the 8 XCDs, workgroups dealt to them
// round-robin): items ordered (group, feature tile, row tile) and cut into
// 8 contiguous ranges, one per XCD, so each XCD streams about 1/8 of the
// weights and of the activation rows once into its own L2, and the row
// tiles that share a weight tile run side by side (2-4% faster than dealing
// items round-robin, measured on the 16384-token prefill).  Router logits
// (K slices) and small grids: item w, w + G, ... of (row tile, feature
// tile[, K slice]).
template <int TBM>
constexpr size_t tile_lds_bytes() {
    return (size_t)n_stages<TBM>() * (TBM + WR) * BK * sizeof(f16);
}

template <int TBM, int NM, int EPI, bool GATHER, bool FR, bool CB>
__global__ __launch_bounds__(kThreads) void tiled_gemm_kernel(StreamArgs a, int n_ntiles,
                                                              int n_groups) {
    extern __shared__ __attribute__((aligned(16))) f16 lds[];
    f16 *As = lds;                                           // [stages][TBM][BK]
    f16 *Bs = lds + n_stages<TBM>() * TBM * BK;              // [stages][WR][BK]
    __shared__ int tstart[kMaxGroups + 1];  // first row tile of each group
    __shared__ int scan[2][kThreads];

    const int tid = threadIdx.x;
    // tiles per group, then an exclusive scan over groups (chunks of 256)
    int carry = 0;
    for (int g0 = 0; g0 < n_groups; g0 += kThreads) {
        const int g = g0 + tid;
        int nt_g = 0;
        if (g < n_groups) {
            int rows = a.offsets ? a.offsets[g + 1] - a.offsets[g] : a.rows_per_group;
            nt_g = rows > 0 ? (rows + TBM - 1) / TBM : 0;
        }
        int cur = 0;
        scan[0][tid] = nt_g;
        __syncthreads();
        for (int o = 1; o < kThreads; o <<= 1) {
            scan[cur ^ 1][tid] = scan[cur][tid] + (tid >= o ? scan[cur][tid - o] : 0);
            cur ^= 1;
            __syncthreads();
        }
        if (g < n_groups) tstart[g] = carry + scan[cur][tid] - nt_g;
        carry += scan[cur][kThreads - 1];
        __syncthreads();
    }
    if (tid == 0) tstart[n_groups] = carry;
    __syncthreads();
    const int ks = EPI == 2 ? a.ksplit : 1;  // K slices (logits only)
    const int total = carry * n_ntiles * ks;

    ItemSeq seq;
    if (EPI != 2 && gridDim.x % 8 == 0) {
        const int xcd = blockIdx.x & 7, nl = gridDim.x >> 3;
        seq.first = (int)((long)total * xcd / 8) + (int)(blockIdx.x >> 3);
        seq.step = nl;
        seq.end = (int)((long)total * (xcd + 1) / 8);
        seq.chunked = true;
    } else {
        seq.first = blockIdx.x;
        seq.step = gridDim.x;
        seq.end = total;
        seq.chunked = false;
    }
    run_items_dma<TBM, NM, EPI, GATHER, FR>(a, As, Bs, tstart, n_groups, n_ntiles, ks, seq);
    if constexpr (CB) {
        static_assert(TBM == kExpertRows && NM == 1 && EPI == 0 && !GATHER, "down projection only");
        static_assert(kCombLds <= tile_lds_bytes<TBM>(), "the combine reuses the stage buffers");
        comb_tail<TBM>(a, seq, tstart, n_groups, n_ntiles, lds);
    }
}

// Per kernel and device, once: allow the kernel's dynamic LDS size and
// count the workgroups that are resident at once (cached; a race only
// repeats the queries; the release store orders the attribute call before
// any thread that reads the cached count launches).
template <int TBM, int NM, int EPI, bool GATHER, bool FR, bool CB>
hipError_t resident_slots(int dev, int &slots) {
    static std::atomic<int> resident[kMaxDevices];
    slots = dev < kMaxDevices ? resident[dev].load(std::memory_order_acquire) : 0;
    if (slots > 0) return hipSuccess;
    const size_t lds = tile_lds_bytes<TBM>();
    hipError_t e = hipFuncSetAttribute((const void *)tiled_gemm_kernel<TBM, NM, EPI, GATHER, FR, CB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int cus = 256, per_cu = 1;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, tiled_gemm_kernel<TBM, NM, EPI, GATHER, FR, CB>, kThreads, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    slots = cus * per_cu;
    if (dev < kMaxDevices) resident[dev].store(slots, std::memory_order_release);
    return hipSuccess;
}

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    return dev;
}

// max_tiles bounds the 128-row tiles (so also the taller ones): it only
// sizes the grid, surplus workgroups find no item and exit.
template <int TBM, int NM, int EPI, bool GATHER, bool FR, bool CB = false>
hipError_t launch_t(const StreamArgs &a, int n_groups, long max_tiles, hipStream_t s) {
    if (n_groups <= 0 || n_groups > kMaxGroups) return hipErrorInvalidValue;
    const int n_ntiles = (a.N + WR / NM - 1) / (WR / NM);
    int slots = 0;
    const hipError_t e = resident_slots<TBM, NM, EPI, GATHER, FR, CB>(current_device(), slots);
    if (e != hipSuccess) return e;
    // every resident workgroup slot, never more than the items
    long grid = slots;
    const long items = max_tiles * n_ntiles * (EPI == 2 ? a.ksplit : 1);
    if (items < grid) grid = items > 0 ? items : 1;
    hipLaunchKernelGGL((tiled_gemm_kernel<TBM, NM, EPI, GATHER, FR, CB>), dim3((unsigned)grid), dim3(kThreads),
                       tile_lds_bytes<TBM>(), s, a, n_ntiles, n_groups);
    return hipGetLastError();
}

}  // namespace

bool tiled_gemm_supported_shape(int K, int dtype, int x_dtype) {
    return dtype == DT_F16 && x_dtype == DT_F16 && K % (2 * BK) == 0;
}

bool tiled_gemm_supported(const StreamArgs &a, int dtype, int x_dtype) {
    return a.ksplit >= 1 && a.K % (2 * BK * a.ksplit) == 0 && a.n_sec == 0 &&
           tiled_gemm_supported_shape(a.K, dtype, x_dtype);
}

hipError_t tiled_gemm_prepare() {
    static std::atomic<bool> ready[kMaxDevices];
    const int dev = current_device();
    if (dev < kMaxDevices && ready[dev].load(std::memory_order_acquire)) return hipSuccess;
    constexpr int XB = kExpertRows;
    int n = 0;
    hipError_t e = hipSuccess;
    // every kernel launch_tiled_gemm can pick
    auto step = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
    };
    step(resident_slots<XB, 2, 1, true, true, false>(dev, n));
    step(resident_slots<XB, 2, 1, false, true, false>(dev, n));
    step(resident_slots<XB, 2, 1, true, false, false>(dev, n));
    step(resident_slots<XB, 2, 1, false, false, false>(dev, n));
    step(resident_slots<XB, 1, 0, false, true, true>(dev, n));
    step(resident_slots<XB, 1, 0, false, false, true>(dev, n));
    step(resident_slots<XB, 1, 0, false, true, false>(dev, n));
    step(resident_slots<XB, 1, 0, false, false, false>(dev, n));
    step(resident_slots<kTiledRouterRows, 1, 2, false, false, false>(dev, n));
    if (e == hipSuccess && dev < kMaxDevices) ready[dev].store(true, std::memory_order_release);
    return e;
}

hipError_t launch_tiled_gemm(const StreamArgs &a, int mode, int n_groups, long max_tiles,
                             hipStream_t s) {
    constexpr int XB = kExpertRows;
    if (a.w_frag && a.N % 16 != 0) return hipErrorInvalidValue;
    if (mode == STREAM_SWIGLU) {
        if (a.w_frag)
            return a.gather ? launch_t<XB, 2, 1, true, true>(a, n_groups, max_tiles, s)
                            : launch_t<XB, 2, 1, false, true>(a, n_groups, max_tiles, s);
        return a.gather ? launch_t<XB, 2, 1, true, false>(a, n_groups, max_tiles, s)
                        : launch_t<XB, 2, 1, false, false>(a, n_groups, max_tiles, s);
    }
    if (mode == STREAM_STORE) {
        if (a.comb.out) {
            // the combine rides in the tail (fp16 rows, top-K within the
            // row lists' room)
            if (a.comb.K < 1 || a.comb.K > kCombMaxK || a.comb.T < 1 || !a.comb.tickets ||
                !a.comb.perm_src || !a.offsets)
                return hipErrorInvalidValue;
            return a.w_frag ? launch_t<XB, 1, 0, false, true, true>(a, n_groups, max_tiles, s)
                            : launch_t<XB, 1, 0, false, false, true>(a, n_groups, max_tiles, s);
        }
        return a.w_frag ? launch_t<XB, 1, 0, false, true>(a, n_groups, max_tiles, s)
                        : launch_t<XB, 1, 0, false, false>(a, n_groups, max_tiles, s);
    }
    // router weights are row-major
    return launch_t<kTiledRouterRows, 1, 2, false, false>(a, n_groups, max_tiles, s);
}

}  // namespace moe
