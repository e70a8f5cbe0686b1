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
// Tile: 128 rows x 256 weight rows (128 features x gate and up for SwiGLU,
// 256 features otherwise), BK = 64.  512 threads = 8 waves (2 per SIMD) in a
// 2 x 4 arrangement; each wave owns 64 rows x 64 weight rows as 16 tiles of
// v_mfma_f32_16x16x32_f16.
// Global -> register -> LDS staging (two register sets), three LDS stages so
// the next step's first fragments are read before the barrier, one barrier
// per K step, XOR-swizzled LDS rows (see swz()).
//
// The grid is persistent (all resident workgroup slots): see tiled_gemm_kernel;
// a workgroup's items share one pipeline where rows are not gathered (see
// run_items).
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128;              // x rows per tile
constexpr int WNW = 4;               // waves along the weight rows (2 x 4 waves)
constexpr int WR = 64 * WNW;         // weight rows per tile (gate + up halves for SwiGLU)
constexpr int BK = 64;               // reduction per pipeline step
constexpr int PITCH = BK;            // halves per LDS row (128 B, XOR-swizzled chunks)
constexpr int kThreads = 128 * WNW;  // 2 x WNW waves
constexpr int RSTEP = kThreads / 8;  // rows one staging pass covers
constexpr int NXL = BM / RSTEP;      // x loads per thread per K step
constexpr int NWL = WR / RSTEP;      // weight loads per thread per K step
constexpr int NSTAGE = 3;            // LDS stages
constexpr int kMaxDevices = 64;

// LDS offset (halves) of 16-byte chunk c of row r: the chunk index is XORed
// with r % 8, so the 16 rows one MFMA fragment read touches spread over all
// banks (a 16-byte row pad still leaves 2-way conflicts on gfx950, as
// measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz(int r, int c) { return r * PITCH + ((c ^ (r & 7)) << 3); }

// One work item: x rows [rs, rs+128) of group g x features [n0, n0 + WR/NM),
// K slice kz (router logits only).  Everything a load or the epilogue needs.
template <int NM>
struct Item {
    int rs, r1, n0, kz, k0;                // rows, features, K slice, K offset
    __amdgpu_buffer_rsrc_t xres, wres[NM];  // this tile's x rows and weight rows
    const f16 *xgat[NXL];                  // gathered x rows (GATHER)
};

template <int NM, int EPI, bool GATHER>
__device__ __forceinline__ Item<NM> make_item(const StreamArgs &a, int g, int mt, int nt, int kz,
                                              int nk) {
    constexpr int FN = WR / NM;  // features per tile
    // wave-uniform by construction; readfirstlane keeps them (and the buffer
    // descriptors built from them) in scalar registers
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
    it.rs = r0 + mt * BM;
    it.r1 = r1;
    it.n0 = nt * FN;
    it.kz = kz;
    it.k0 = EPI == 2 ? kz * nk * BK : 0;
    const int K = a.K;
    const int tid = threadIdx.x;
    // Buffer loads against per-tile resource descriptors: rows past the
    // tile's valid rows fall outside the descriptor's range and load zeros,
    // so no clamping is needed; 32-bit lane offsets keep the address cost at
    // one VGPR per load.
    const int rows_valid = (r1 - it.rs) < BM ? (r1 - it.rs) : BM;
    const int xrow0 = a.x_broadcast ? it.rs - r0 : it.rs;
    it.xres = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const f16 *>(a.x) + (size_t)xrow0 * K), (short)0,
        rows_valid * K * 2, 0x00020000);
    // gathered x rows (rows named by a.gather): plain global loads from the
    // row each thread moves; rows past the group repeat its last row (never
    // stored)
    if (GATHER) {
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            int r = it.rs + (tid >> 3) + RSTEP * i;
            if (r > r1 - 1) r = r1 - 1;
            it.xgat[i] = reinterpret_cast<const f16 *>(a.x) +
                         (size_t)(a.gather[r] / a.gather_div) * K + (tid & 7) * 8;
        }
    }
    const int ncols = (a.N - it.n0) < FN ? (a.N - it.n0) : FN;
#pragma unroll
    for (int m = 0; m < NM; ++m)
        it.wres[m] = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(reinterpret_cast<const f16 *>(m == 0 ? a.w0 : a.w1) +
                     (size_t)g * a.w_group_stride + (size_t)it.n0 * K),
            (short)0, ncols * K * 2, 0x00020000);
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

// The items of one workgroup, one after the other, with one pipeline: the
// loads of an item's first K steps are issued during the previous item's
// last steps (its K steps past the end map to the next item's first ones),
// so only the workgroup's first item starts by waiting for memory.
// 8 waves = 2 (rows) x 4 (weight rows); wave (wm, wn) owns x rows
// wm*64..+64 and, per matrix m, weight rows m*FN + wn*FN/4 .. +FN/4
// (FN = WR/NM features), as 4 x (4/NM) x NM tiles of 16x16x32 MFMAs.
template <int NM, int EPI, bool GATHER>
__device__ __forceinline__ void run_items(const StreamArgs &a, f16 *As, f16 *Bs,
                                          const int *tstart, int n_groups, int n_ntiles, int ks,
                                          const ItemSeq seq) {
    constexpr int FN = WR / NM;   // features per tile
    constexpr int NJ = 4 / NM;    // 16-feature subtiles per wave and matrix
    const int K = a.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WNW, wn = wave % WNW;
    const int lr = lane & 15, lg = lane >> 4;
    // K steps per item: [kz*nk, (kz+1)*nk), nk even (K is a multiple of
    // 2*BK*ksplit).  Items chain only with nk >= 4 (the loads run up to 3
    // steps ahead), and not when x rows are gathered (the next item's row
    // indices would be waited for together with the in-flight staging
    // loads: measured 1% slower); otherwise each item restarts the pipeline.
    const int nk = EPI == 2 ? K / BK / a.ksplit : K / BK;
    constexpr bool CHAIN = !GATHER;
    const bool chain = CHAIN && nk >= 4;

    // Thread t moves 16-byte chunk t%8 of rows t/8 + RSTEP*i (i < NXL for x,
    // i < NWL for the weight rows).
    const int trow = tid >> 3, tch = tid & 7;
    const int goff = trow * K * 2 + tch * 16;  // byte offset of row trow, chunk tch
    const int rstep = RSTEP * K * 2;           // RSTEP rows further
    const int lds0 = swz(trow, tch);           // (trow + RSTEP i) % 8 == trow % 8

    // two register staging sets: set 0 holds even K steps, set 1 odd ones
    f16x8 ra0[NXL], rb0[NWL], ra1[NXL], rb1[NWL];
    // K step s of the chain: steps past the current item's end belong to the
    // next item (or re-read the last step when there is none; never used).
    // Branch-free (scalar selects), so the compiler's wait counts stay exact.
    auto gload = [&](f16x8 *RA, f16x8 *RB, const Item<NM> &cur, const Item<NM> &nxt,
                     bool has_nxt, int s) {
        const bool to_nxt = CHAIN && s >= nk && has_nxt;
        const int sk = s < nk ? s : (to_nxt ? s - nk : nk - 1);
        const int kb = ((to_nxt ? nxt.k0 : cur.k0) + sk * BK) * 2;
        if (GATHER) {
#pragma unroll
            for (int i = 0; i < NXL; ++i)
                RA[i] = load16((to_nxt ? nxt.xgat[i] : cur.xgat[i]) + kb / 2);
        } else {
            const __amdgpu_buffer_rsrc_t xr = to_nxt ? nxt.xres : cur.xres;
#pragma unroll
            for (int i = 0; i < NXL; ++i)
                RA[i] = __builtin_bit_cast(
                    f16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, goff + i * rstep + kb, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < NWL; ++i) {
            const int m = (i * RSTEP) / FN;
            const __amdgpu_buffer_rsrc_t wr = to_nxt ? nxt.wres[m] : cur.wres[m];
            RB[i] = __builtin_bit_cast(
                f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                           wr, goff + ((i * RSTEP) % FN / RSTEP) * rstep + kb, 0, 0));
        }
    };
    auto lstore = [&](const f16x8 *RA, const f16x8 *RB, int st) {
        f16 *A_ = As + st * BM * PITCH + lds0;
        f16 *B_ = Bs + st * WR * PITCH + lds0;
#pragma unroll
        for (int i = 0; i < NXL; ++i) *reinterpret_cast<f16x8 *>(A_ + i * RSTEP * PITCH) = RA[i];
#pragma unroll
        for (int i = 0; i < NWL; ++i) *reinterpret_cast<f16x8 *>(B_ + i * RSTEP * PITCH) = RB[i];
    };

    // Three LDS stages: step k computes from stage k%3 while the staged data
    // of step k+2 goes to stage (k+2)%3 (last read during step k-1), so the
    // first-half fragments of step k+1 (stage (k+1)%3, complete since the
    // barrier that ended step k-1) are read during step k and no step starts
    // by waiting for LDS.  Per step: the 16 MFMAs of the first K half with
    // the fragment reads of the second, then the 16 of the second half with
    // the next step's first-half reads, the staging writes and the refill
    // loads, pinned with scheduling-group barriers; one barrier per step.
    f16x8 af0[4], bf0[NM][NJ], af1[4], bf1[NM][NJ];
    auto fread = [&](f16x8 *af, f16x8 (*bf)[NJ], int st, int kq) {
        const f16 *A = As + st * BM * PITCH;
        const f16 *B = Bs + st * WR * PITCH;
        const int ch = kq + lg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const f16x8 *>(A + swz(wm * 64 + i * 16 + lr, ch));
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                bf[m][j] = *reinterpret_cast<const f16x8 *>(
                    B + swz(m * FN + wn * (FN / WNW) + j * 16 + lr, ch));
    };
    f32x4 acc[NM][4][NJ];
    auto mm = [&](const f16x8 *af, f16x8 (*bf)[NJ]) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[m][i][j] = mfma16(af[i], bf[m][j], acc[m][i][j]);
    };
    auto order = [&]() {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int r = 0; r < NXL + NWL; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8 - NXL - NWL, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    if (seq.first >= seq.end) return;
    int g, mt, nt, kz;
    decode_item(tstart, n_groups, n_ntiles, ks, seq.chunked, seq.first, g, mt, nt, kz);
    Item<NM> cur = make_item<NM, EPI, GATHER>(a, g, mt, nt, kz, nk);
    Item<NM> nxt = cur;
    int inext = seq.first + seq.step;
    bool primed = false;  // the pipeline already holds this item's first steps
    int s0 = 0, s1 = 1, s2 = 2;  // stages of steps kt, kt+1, kt+2
    for (;;) {
        const bool has_nxt = chain && inext < seq.end;
        if (has_nxt) {
            decode_item(tstart, n_groups, n_ntiles, ks, seq.chunked, inext, g, mt, nt, kz);
            nxt = make_item<NM, EPI, GATHER>(a, g, mt, nt, kz, nk);
        }
        if (!primed) {
            gload(ra0, rb0, cur, nxt, false, 0);
            gload(ra1, rb1, cur, nxt, false, 1);
            lstore(ra0, rb0, s0);
            lstore(ra1, rb1, s1);
            gload(ra0, rb0, cur, nxt, has_nxt, 2);
            __syncthreads();
            fread(af0, bf0, s0, 0);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kt = 0; kt < nk; kt += 2) {
            fread(af1, bf1, s0, 4);
            mm(af0, bf0);
            fread(af0, bf0, s1, 0);
            mm(af1, bf1);
            lstore(ra0, rb0, s2);
            gload(ra1, rb1, cur, nxt, has_nxt, kt + 3);
            order();
            fread(af1, bf1, s1, 4);
            mm(af0, bf0);
            fread(af0, bf0, s2, 0);
            mm(af1, bf1);
            lstore(ra1, rb1, s0);
            gload(ra0, rb0, cur, nxt, has_nxt, kt + 4);
            order();
            // steps kt+2, kt+3, kt+4 sit in stages s2, s0, s1
            const int t = s0;
            s0 = s2;
            s2 = s1;
            s1 = t;
        }

        // ---- epilogue.  acc[m][i][j]: x row wm*64 + i*16 + 4*lg + q
        // (q = 0..3), feature n0 + wn*FN/4 + j*16 + lr (A = x rows, B =
        // weight rows).
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = cur.rs + wm * 64 + i * 16 + 4 * lg + q;
                if (r >= cur.r1) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int f = cur.n0 + wn * (FN / WNW) + j * 16 + lr;
                    if (f >= a.N) continue;
                    if (EPI == 2) {  // logits, fp32 partial of K slice kz
                        reinterpret_cast<float *>(a.out)[(size_t)cur.kz * a.split_stride +
                                                         (size_t)r * a.out_ld + f] =
                            acc[0][i][j][q];
                    } else {
                        float v;
                        if (EPI == 1)
                            v = siluf_(acc[0][i][j][q]) * acc[NM - 1][i][j][q];
                        else
                            v = acc[0][i][j][q];
                        reinterpret_cast<f16 *>(a.out)[(size_t)r * a.out_ld + f] = to_f16(v);
                    }
                }
            }
        }
        if (!has_nxt && inext >= seq.end) break;
        // the next item: chained (its first steps are already staged, its
        // first fragments read) or restarted
        primed = has_nxt;
        if (!has_nxt) {
            // restart: every stage is free (the last step's barrier came
            // after every fragment read)
            decode_item(tstart, n_groups, n_ntiles, ks, seq.chunked, inext, g, mt, nt, kz);
            nxt = make_item<NM, EPI, GATHER>(a, g, mt, nt, kz, nk);
            s0 = 0;
            s1 = 1;
            s2 = 2;
        }
        cur = nxt;
        inext += seq.step;
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
template <int NM, int EPI, bool GATHER>
__global__ __launch_bounds__(kThreads) void tiled_gemm_kernel(StreamArgs a, int n_ntiles,
                                                              int n_groups) {
    extern __shared__ __attribute__((aligned(16))) f16 lds[];
    f16 *As = lds;                          // [NSTAGE][BM][PITCH]
    f16 *Bs = lds + NSTAGE * BM * PITCH;    // [NSTAGE][WR][PITCH]
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
            nt_g = rows > 0 ? (rows + BM - 1) / BM : 0;
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
    run_items<NM, EPI, GATHER>(a, As, Bs, tstart, n_groups, n_ntiles, ks, seq);
}

template <int NM, int EPI, bool GATHER>
hipError_t launch_t(const StreamArgs &a, int n_groups, long max_tiles, hipStream_t s) {
    if (n_groups <= 0 || n_groups > kMaxGroups) return hipErrorInvalidValue;
    const int n_ntiles = (a.N + WR / NM - 1) / (WR / NM);
    const size_t lds = (size_t)NSTAGE * (BM + WR) * PITCH * sizeof(f16);
    // Per device, once: allow the dynamic LDS size and count the workgroups
    // that are resident at once (cached; a race only repeats the queries).
    static std::atomic<int> resident[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int slots = dev < kMaxDevices ? resident[dev].load(std::memory_order_relaxed) : 0;
    if (slots <= 0) {
        hipError_t e = hipFuncSetAttribute((const void *)tiled_gemm_kernel<NM, EPI, GATHER>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        int cus = 256, per_cu = 1;
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, tiled_gemm_kernel<NM, EPI, GATHER>, kThreads, lds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        slots = cus * per_cu;
        if (dev < kMaxDevices) resident[dev].store(slots, std::memory_order_relaxed);
    }
    // every resident workgroup slot, never more than the items
    long grid = slots;
    const long items = max_tiles * n_ntiles * (EPI == 2 ? a.ksplit : 1);
    if (items < grid) grid = items > 0 ? items : 1;
    hipLaunchKernelGGL((tiled_gemm_kernel<NM, EPI, GATHER>), dim3((unsigned)grid), dim3(kThreads),
                       lds, s, a, n_ntiles, n_groups);
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

hipError_t launch_tiled_gemm(const StreamArgs &a, int mode, int n_groups, long max_tiles,
                             hipStream_t s) {
    if (mode == STREAM_SWIGLU)
        return a.gather ? launch_t<2, 1, true>(a, n_groups, max_tiles, s)
                        : launch_t<2, 1, false>(a, n_groups, max_tiles, s);
    if (mode == STREAM_STORE) return launch_t<1, 0, false>(a, n_groups, max_tiles, s);
    return launch_t<1, 2, false>(a, n_groups, max_tiles, s);
}

}  // namespace moe
