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
// Tile: BM = 128 rows x BN = 128 features (x2 weight matrices for SwiGLU),
// BK = 64.  256 threads = 4 waves in a 2 x 2 arrangement; each wave owns a
// 64 x 64 block (x2 matrices) as 4 x 4 tiles of v_mfma_f32_16x16x32_f16.
// Global -> register -> LDS staging, two LDS buffers, one barrier per K step;
// LDS rows are padded by 16 bytes so the 16-byte fragment reads of 16
// different rows fall in different banks.
//
// The grid is persistent (one workgroup per CU): see tiled_gemm_kernel.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int PITCH = BK + 8;  // halves per LDS row (16 B pad)
constexpr int kThreads = 256;

template <int NM, int EPI>
__device__ __forceinline__ void tile_body(const StreamArgs &a, f16 *As, f16 *Bs, int g, int mt,
                                          int nt) {
    int r0, r1;
    if (a.offsets) {
        r0 = a.offsets[g];
        r1 = a.offsets[g + 1];
    } else {
        r0 = g * a.rows_per_group;
        r1 = r0 + a.rows_per_group;
    }
    const int rs = r0 + mt * BM;
    const int n0 = nt * BN;
    const int K = a.K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves
    const int lr = lane & 15, lg = lane >> 4;

    // ---- global load assignment: 16-byte chunks, 8 per 128-byte row slice
    // A: BM rows x 8 chunks = 1024 chunks -> 4 per thread
    // B: NM*BN rows x 8 chunks -> 4*NM per thread
    const f16 *xg[4];
    int a_lds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + kThreads * i;
        const int row = c >> 3, col = (c & 7) * 8;
        int r = rs + row;
        if (r > r1 - 1) r = r1 - 1;
        const int xr = a.x_broadcast ? r - r0 : r;
        xg[i] = reinterpret_cast<const f16 *>(a.x) + (size_t)xr * K + col;
        a_lds[i] = row * PITCH + col;
    }
    const f16 *wg[4 * NM];
    int b_lds[4 * NM];
#pragma unroll
    for (int i = 0; i < 4 * NM; ++i) {
        const int c = tid + kThreads * i;
        const int row = c >> 3, col = (c & 7) * 8;  // row in [0, NM*BN)
        const int m = row / BN, rr = row % BN;
        int n = n0 + rr;
        if (n > a.N - 1) n = a.N - 1;
        const f16 *base = reinterpret_cast<const f16 *>(m == 0 ? a.w0 : a.w1);
        wg[i] = base + (size_t)g * a.w_group_stride + (size_t)n * K + col;
        b_lds[i] = row * PITCH + col;
    }

    f16x8 ra[4], rb[4 * NM];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = load16(xg[i] + k0);
#pragma unroll
        for (int i = 0; i < 4 * NM; ++i) rb[i] = load16(wg[i] + k0);
    };
    auto lstore = [&](int buf) {
        f16 *A = As + buf * BM * PITCH;
        f16 *B = Bs + buf * NM * BN * PITCH;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<f16x8 *>(A + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < 4 * NM; ++i) *reinterpret_cast<f16x8 *>(B + b_lds[i]) = rb[i];
    };

    f32x4 acc[NM][4][4];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const f16 *A = As + buf * BM * PITCH;
        const f16 *B = Bs + buf * NM * BN * PITCH;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            f16x8 af[4], bf[NM][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const f16x8 *>(A + (wm * 64 + i * 16 + lr) * PITCH + ks + lg * 8);
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bf[m][j] = *reinterpret_cast<const f16x8 *>(
                        B + (m * BN + wn * 64 + j * 16 + lr) * PITCH + ks + lg * 8);
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[m][i][j] = mfma16(af[i], bf[m][j], acc[m][i][j]);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  acc[m][i][j]: rows wm*64 + i*16 + 4*lg + q (q = 0..3),
    // feature n0 + wn*64 + j*16 + lr (A = x rows, B = weight rows).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rs + wm * 64 + i * 16 + 4 * lg + q;
            if (r >= r1) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int f = n0 + wn * 64 + j * 16 + lr;
                if (f >= a.N) continue;
                if (EPI == 2) {  // logits, fp32
                    reinterpret_cast<float *>(a.out)[(size_t)r * a.out_ld + f] = acc[0][i][j][q];
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
}

constexpr int kMaxGroups = 1024;

// Persistent: a fixed grid walks the real tiles.  Each workgroup first builds
// the prefix of row tiles per group from the device-side offsets (group
// sizes are only known on the device), then takes items w, w + G, ...
// Items are ordered (group, row tile, feature tile), feature tile fastest;
// with 8 XCDs dealt round-robin and a multiple-of-8 feature-tile count, all
// row tiles of one (group, feature tile) land on the same XCD, so that
// weight tile is reused from its L2.
template <int NM, int EPI>
__global__ __launch_bounds__(kThreads) void tiled_gemm_kernel(StreamArgs a, int n_ntiles,
                                                              int n_groups) {
    extern __shared__ __attribute__((aligned(16))) f16 lds[];
    f16 *As = lds;                          // [2][BM][PITCH]
    f16 *Bs = lds + 2 * BM * PITCH;         // [2][NM*BN][PITCH]
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
    const int total = carry * n_ntiles;

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int tile = item / n_ntiles;
        const int nt = item % n_ntiles;
        // group holding this row tile: last g with tstart[g] <= tile
        int lo = 0, hi = n_groups - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tstart[mid] <= tile)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int g = lo;
        const int mt = tile - tstart[g];
        tile_body<NM, EPI>(a, As, Bs, g, mt, nt);
    }
}

template <int NM, int EPI>
hipError_t launch_t(const StreamArgs &a, int n_groups, long max_tiles, hipStream_t s) {
    if (n_groups <= 0 || n_groups > kMaxGroups) return hipErrorInvalidValue;
    const int n_ntiles = (a.N + BN - 1) / BN;
    const size_t lds = (size_t)2 * (BM + NM * BN) * PITCH * sizeof(f16);
    static bool attr_set = false;  // idempotent; a race only repeats the call
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)tiled_gemm_kernel<NM, EPI>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    // one resident workgroup per CU (LDS-bound); never more than the items
    long grid = cus;
    const long items = max_tiles * n_ntiles;
    if (items < grid) grid = items > 0 ? items : 1;
    hipLaunchKernelGGL((tiled_gemm_kernel<NM, EPI>), dim3((unsigned)grid), dim3(kThreads), lds, s,
                       a, n_ntiles, n_groups);
    return hipGetLastError();
}

}  // namespace

bool tiled_gemm_supported(const StreamArgs &a, int dtype, int x_dtype) {
    return dtype == DT_F16 && x_dtype == DT_F16 && a.ksplit == 1 && a.K % BK == 0;
}

hipError_t launch_tiled_gemm(const StreamArgs &a, int mode, int n_groups, long max_tiles,
                             hipStream_t s) {
    if (mode == STREAM_SWIGLU) return launch_t<2, 1>(a, n_groups, max_tiles, s);
    if (mode == STREAM_STORE) return launch_t<1, 0>(a, n_groups, max_tiles, s);
    return launch_t<1, 2>(a, n_groups, max_tiles, s);
}

}  // namespace moe
