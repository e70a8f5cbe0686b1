// gemm_stream.hip -- grouped "weight-stream" GEMM on MFMA for small row counts.
//
// Serves the router linear (Step 1 of the expert-parallelism blog page,
// section 2.2) and both halves of the SwiGLU expert FFN (Step 3) when each
// group (expert slot) holds few rows, i.e. decode.  There the work is bound by
// reading every touched weight byte once from HBM (the decode-is-memory-bound
// analysis of the PPIO essay on EP), so the kernel streams weights straight
// from HBM into registers and never stages them in LDS:
//
//   out[r][n] = epilogue( sum_k W[g][n][k] * x[r][k] )   for rows r of group g
//
// Work decomposition
//   blockIdx.x  a block of features: 4 waves x 16*NSUB features each (KW = 1),
//               or 16*NSUB = 64 features shared by the 4 waves (KW = 4: the
//               expert GEMMs, and the fp16 router when its K slices are
//               multiples of 512; SwiGLU reads a gate and an up tile per
//               16-feature subtile)
//   blockIdx.y  group g (expert slot)
//   blockIdx.z  (first row block) * ksplit + K slice; row blocks of 64 rows
//               are strided by gridDim.z / ksplit.  ksplit > 1 (router only)
//               writes one fp32 partial per K slice; the top-K kernel sums
//               them in slice order, so the result stays deterministic.
// KW = 4: wave w of a block runs quarter w of K (of the K slice, for the
// router) for all 64 features, so each activation fragment it loads feeds 4
// (down, router) or 8 (gate/up) MFMAs and a block loads its token rows once,
// while a block still covers only 64 features (fine-grained blocks keep the
// tail of an uneven grid short).  The 4 partial tiles meet
// in LDS and are summed in K order (deterministic); wave w then applies the
// epilogue to subtile w.  The 64 rows of a row block are processed in MT =
// 1, 2 or 4 tiles of 16, chosen from the rows actually present, so one pass
// over the weights serves every row of a decode-sized group.
//
// MFMA mapping (v_mfma_f32_16x16x32_f16, or 4x v_mfma_f32_16x16x4_f32 for
// fp32): A = 16 weight rows (features), B = x^T (16 rows = tokens).  Lane l
// reads 16 contiguous bytes of weight row l%16 and of token row l%16 at the
// same K offset.  With row-major weights a wave instruction covers 16 rows x
// 64 bytes and two consecutive K chunks cover whole 128-byte lines; with
// weights in the fragment layout (frag_offset) the same 16 x 64 bytes are
// one contiguous 1 KB, and those loads carry the nontemporal hint (every
// weight byte is read once).  Measured on MI355X, the fragment layout with
// the hint streams the gate/up weights about 11% faster than row-major
// loads (about 6.9 against 6.2 TB/s); the hint on row-major loads, whose
// two halves of a 128-byte line come from two instructions, is slower
// instead.  Loads are double buffered in registers, U chunks per buffer, to
// keep several KB per wave in flight against HBM latency.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Kernel shapes (measured best on MI355X, fragment-layout weights):
//   kU              K chunks per register buffer (double-buffered) of the
//                   one-wave-per-slice shapes
//   kStoreWideRows  expected rows per group from which the plain (down
//                   projection) GEMM takes the wide shape (one subtile per
//                   wave is faster at 4 and 8 rows per group, the wide shape
//                   at 15)
//   kStoreNsubWide, kStoreUWide  subtiles per wave and K chunks per buffer
//                   of that wide shape
//   kSwigluNsub, kSwigluU  the SwiGLU GEMM's subtiles and chunks per buffer
//   kSwigluUFp8     chunks per buffer when x is fp8 codes (the decode VALU
//                   work per chunk makes one chunk per buffer ~1% faster)
// The wide store shape, the SwiGLU GEMM and the fp16 router split K over
// the 4 waves of a block (KW = 4) when K allows it.
constexpr int kU = 8;
constexpr int kStoreWideRows = 12;
constexpr int kStoreNsubWide = 4;
constexpr int kStoreUWide = 2;
constexpr int kSwigluNsub = 4;
constexpr int kSwigluU = 2;
constexpr int kSwigluUFp8 = 1;

// Epilogues
enum : int { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_LOGITS = 2 };

template <typename TW, int XM>
struct XFrag {  // raw x fragment as loaded (same dtype as W)
    typedef typename Frag<TW>::vec raw;
    __device__ static __forceinline__ raw load(const void *base, size_t elem) {
        return load16(reinterpret_cast<const TW *>(base) + elem);
    }
    __device__ static __forceinline__ typename Frag<TW>::vec cvt(const raw &v) { return v; }
};
template <>
struct XFrag<f16, DT_FP8> {  // 8 fp8 codes, decoded to fp16 * 2^-8
    typedef u32x2 raw;
    __device__ static __forceinline__ raw load(const void *base, size_t elem) {
        return *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint8_t *>(base) + elem);
    }
    __device__ static __forceinline__ f16x8 cvt(const raw &v) { return e4m3x8_to_f16x8_scaled(v); }
};

// Weight loads: every weight byte is read exactly once per launch; NT marks
// the load nontemporal (fragment layout only, see above).
template <bool NT, typename T>
__device__ __forceinline__ typename Frag<T>::vec wload16(const T *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const typename Frag<T>::vec *>(p));
    else
        return load16(p);
}

// NSUB 16-feature subtiles per wave; NM = weight tiles per K chunk (SwiGLU:
// gate subtiles 0..NSUB-1, then the up subtiles; otherwise NM = NSUB).
// FR: weights in the fragment layout (N a multiple of 16).
// KW == 1: the wave runs K slice kz of ksplit and finishes its features.
// KW == 4: the block's 4 waves share the same NSUB = 4 subtiles, wave w
// runs quarter w of K; the partials meet in LDS (red) and are summed in K
// order, then wave w finishes subtile w.  Every activation fragment then
// serves 4x as many weight rows while a block still streams 64 features.
template <typename TW, int XM, int NSUB, int EPI, int KW, int MT, int U, bool FR>
__device__ __forceinline__ void stream_pass(const StreamArgs &a, int g, int f0, int rstart,
                                            int r0, int r1, int kz, f32x4 *red) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr int NM = SW ? 2 * NSUB : NSUB;
    static_assert(KW == 1 || (KW == 4 && NSUB == 4), "K split shape");
    typedef typename Frag<TW>::vec V;
    typedef XFrag<TW, XM> XF;
    typedef typename XF::raw XR;
    constexpr int EL = Frag<TW>::kElems;  // elements per lane fragment
    constexpr int CK = 4 * EL;            // K covered by one fragment step
    const int lane = lane_id();
    const int lr = lane & 15, lg = lane >> 4;
    const int K = a.K;
    const int wk = KW > 1 ? (int)(threadIdx.x >> 6) : 0;
    const int KS = K / (a.ksplit * KW);  // this wave's K slice: [ksl*KS, (ksl+1)*KS)
    const int ksl = kz * KW + wk;
    const int NC = KS / CK;

    // weight rows (clamped: rows past N are read but never stored).  Tile m
    // covers rows f0 + 16 * (m % NSUB) .. +15 of the gate matrix (w0) for
    // m < NSUB and of the up matrix (w1) above (SwiGLU).  Fragment layout:
    // the tile's first fragment of this K slice; a K chunk is 1 KB further.
    constexpr int WSTEP = FR ? 16 * CK : CK;  // elements from one K chunk to the next
    const TW *wp[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        size_t off;
        if constexpr (FR) {
            int gi = f0 / 16 + (m % NSUB);
            if (gi > a.N / 16 - 1) gi = a.N / 16 - 1;
            off = ((size_t)gi * (K / CK) + (size_t)ksl * (KS / CK)) * (16 * CK) +
                  (size_t)lane * EL;
        } else {
            int wrow = f0 + 16 * (m % NSUB) + lr;
            if (wrow > a.N - 1) wrow = a.N - 1;
            off = (size_t)wrow * K + (size_t)ksl * KS + (size_t)lg * EL;
        }
        wp[m] = reinterpret_cast<const TW *>(m < NSUB ? a.w0 : a.w1) +
                (size_t)g * a.w_group_stride + off;
    }
    // token rows (clamped to the group's last row; extra columns are dropped)
    size_t xo[MT];
    int rows[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int r = rstart + t * 16 + lr;
        rows[t] = r;
        int rc = r < r1 ? r : r1 - 1;
        int xr = a.gather ? a.gather[rc] / a.gather_div : (a.x_broadcast ? rc - r0 : rc);
        xo[t] = (size_t)xr * K + (size_t)ksl * KS + (size_t)lg * EL;
    }

    f32x4 acc[NM][MT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    V wa[U][NM], wb[U][NM];
    XR xa[U][MT], xb[U][MT];

#define MOE_LOAD(WBUF, XBUF, c)                                                  \
    _Pragma("unroll") for (int u = 0; u < U; ++u) {                              \
        _Pragma("unroll") for (int m = 0; m < NM; ++m) WBUF[u][m] =              \
            wload16<FR>(wp[m] + (size_t)((c) + u) * WSTEP);                      \
        _Pragma("unroll") for (int t = 0; t < MT; ++t) XBUF[u][t] =              \
            XF::load(a.x, xo[t] + (size_t)((c) + u) * CK);                       \
    }
#define MOE_COMPUTE(WBUF, XBUF)                                                  \
    _Pragma("unroll") for (int u = 0; u < U; ++u) {                              \
        _Pragma("unroll") for (int t = 0; t < MT; ++t) {                         \
            V xv = XF::cvt(XBUF[u][t]);                                          \
            _Pragma("unroll") for (int m = 0; m < NM; ++m) acc[m][t] =           \
                mfma16(WBUF[u][m], xv, acc[m][t]);                               \
        }                                                                        \
    }

    // Double buffering (NC is a multiple of 2U): buffer b's loads are in
    // flight while buffer a is computed, and the next group of a's while b
    // is.  The last iteration skips the prefetch past the end; the compiler
    // then waits for every outstanding load before that iteration's second
    // compute.
    MOE_LOAD(wa, xa, 0);
    for (int c = 0; c < NC; c += 2 * U) {
        MOE_LOAD(wb, xb, c + U);
        MOE_COMPUTE(wa, xa);
        if (c + 2 * U < NC) MOE_LOAD(wa, xa, c + 2 * U);
        MOE_COMPUTE(wb, xb);
    }
#undef MOE_LOAD
#undef MOE_COMPUTE

    if (KW > 1) {
        // partials of the 4 K quarters -> wave wk finishes subtile wk
#pragma unroll
        for (int t = 0; t < MT; ++t) {
#pragma unroll
            for (int m = 0; m < NM; ++m) red[(wk * NM + m) * 64 + lane] = acc[m][t];
            __syncthreads();
            f32x4 s0 = red[wk * 64 + lane];
            f32x4 s1 = SW ? red[(NSUB + wk) * 64 + lane] : s0;
#pragma unroll
            for (int v = 1; v < KW; ++v) {
                s0 += red[(v * NM + wk) * 64 + lane];
                if (SW) s1 += red[(v * NM + NSUB + wk) * 64 + lane];
            }
            __syncthreads();
            const int r = rows[t];
            if (EPI == EPI_LOGITS) {  // fp32 partial of K slice kz
                if (r < r1) {
                    float *o = reinterpret_cast<float *>(a.out) + (size_t)kz * a.split_stride +
                               (size_t)r * a.out_ld;
                    const int fb = f0 + 16 * wk + 4 * lg;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (fb + j < a.N) o[fb + j] = s0[j];
                }
            } else if (r < r1) {
                float sc = 1.0f;
                if (XM == DT_FP8) sc = a.x_scale[r] * 256.0f;  // undo the 2^-8 of the decode
                const int fb = f0 + 16 * wk + 4 * lg;
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = SW ? siluf_(s0[j] * sc) * (s1[j] * sc) : s0[j] * sc;
                TW *o = reinterpret_cast<TW *>(a.out) + (size_t)r * a.out_ld + fb;
                if (fb < a.N) {
                    if (sizeof(TW) == 2) {
                        f16x4 h4 = {to_f16(v[0]), to_f16(v[1]), to_f16(v[2]), to_f16(v[3])};
                        *reinterpret_cast<f16x4 *>(o) = h4;
                    } else {
                        *reinterpret_cast<f32x4 *>(o) = f32x4{v[0], v[1], v[2], v[3]};
                    }
                }
            }
        }
        return;
    }

    // epilogue: lane holds features f0 (+16m) + 4*lg + j (j = 0..3) of token rows[t]
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int r = rows[t];
        if (r >= r1) continue;
        float sc = 1.0f;
        if (XM == DT_FP8) sc = a.x_scale[r] * 256.0f;  // undo the 2^-8 of the decode
#pragma unroll
        for (int m = 0; m < NSUB; ++m) {  // 16-feature output blocks
            const int fb = f0 + 16 * m + 4 * lg;
            if (EPI == EPI_LOGITS) {
                float *o = reinterpret_cast<float *>(a.out) + (size_t)kz * a.split_stride +
                           (size_t)r * a.out_ld;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int f = fb + j;
                    if (f < a.N) o[f] = acc[m][t][j];
                }
            } else {
                if (fb >= a.N) continue;  // N % 64 == 0 makes this unreachable
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (SW) {
                        const float ga = acc[m][t][j] * sc, ub = acc[NSUB + m][t][j] * sc;
                        v[j] = siluf_(ga) * ub;
                    } else {
                        v[j] = acc[m][t][j] * sc;
                    }
                }
                TW *o = reinterpret_cast<TW *>(a.out) + (size_t)r * a.out_ld + fb;
                if (sizeof(TW) == 2) {
                    f16x4 h4 = {to_f16(v[0]), to_f16(v[1]), to_f16(v[2]), to_f16(v[3])};
                    *reinterpret_cast<f16x4 *>(o) = h4;
                } else {
                    *reinterpret_cast<f32x4 *>(o) = f32x4{v[0], v[1], v[2], v[3]};
                }
            }
        }
    }
}

template <typename TW, int XM, int NSUB, int EPI, int KW, int U, bool FR>
__global__ __launch_bounds__(256) void stream_gemm_kernel(StreamArgs a) {
    constexpr int FPW = 16 * NSUB;  // features per wave
    constexpr int NM = EPI == EPI_SWIGLU ? 2 * NSUB : NSUB;
    __shared__ f32x4 red[KW > 1 ? KW * NM * 64 : 1];
    const int wave = threadIdx.x >> 6;
    const int f0 = KW > 1 ? blockIdx.x * FPW : blockIdx.x * (4 * FPW) + wave * FPW;
    if (f0 >= a.N) return;  // block-uniform when KW > 1
    const int kz = blockIdx.z % a.ksplit;  // K slice
    const int zr = blockIdx.z / a.ksplit;  // first row block
    const int zn = gridDim.z / a.ksplit;   // row-block stride
    int g = blockIdx.y, r0, r1;
    StreamArgs b = a;
    if (g < a.n_sec) {  // secondary uniform group (e.g. a shared expert)
        b.x = a.x2;
        b.x_broadcast = a.x2_broadcast;
        b.gather = nullptr;
        b.w0 = a.w0b;
        b.w1 = a.w1b;
        r0 = a.row2_base + g * a.rows2;
        r1 = r0 + a.rows2;
    } else {
        g -= a.n_sec;
        if (a.offsets) {
            r0 = a.offsets[g];
            r1 = a.offsets[g + 1];
        } else {
            r0 = g * a.rows_per_group;
            r1 = r0 + a.rows_per_group;
        }
    }
    for (int rb = zr; r0 + rb * 64 < r1; rb += zn) {
        const int rs = r0 + rb * 64;
        const int n = r1 - rs;
        constexpr int U2 = U;
        constexpr int U4 = KW > 1 ? 1 : (U > 2 ? 2 : U);
        if (n <= 16)
            stream_pass<TW, XM, NSUB, EPI, KW, 1, U, FR>(b, g, f0, rs, r0, r1, kz, red);
        else if (n <= 32)
            stream_pass<TW, XM, NSUB, EPI, KW, 2, U2, FR>(b, g, f0, rs, r0, r1, kz, red);
        else
            stream_pass<TW, XM, NSUB, EPI, KW, 4, U4, FR>(b, g, f0, rs, r0, r1, kz, red);
    }
}

template <typename TW, int XM, int NSUB, int EPI, int U, int KW, bool FR>
hipError_t launch_l(const StreamArgs &a, int n_groups, int zblocks, hipStream_t s) {
    constexpr int FPB = (KW > 1 ? 1 : 4) * 16 * NSUB;  // features per block
    dim3 grid((a.N + FPB - 1) / FPB, n_groups + a.n_sec, zblocks * a.ksplit);
    constexpr int CK = 4 * Frag<TW>::kElems;
    const int NC = a.K / (a.ksplit * KW) / CK;
    if (a.ksplit < 1 || a.K % (a.ksplit * KW * 4 * CK) != 0) return hipErrorInvalidValue;
    if (FR && a.N % 16 != 0) return hipErrorInvalidValue;
    if (NC % (2 * U) == 0)
        hipLaunchKernelGGL((stream_gemm_kernel<TW, XM, NSUB, EPI, KW, U, FR>), grid, dim3(256), 0,
                           s, a);
    else
        hipLaunchKernelGGL((stream_gemm_kernel<TW, XM, NSUB, EPI, KW, 2, FR>), grid, dim3(256), 0,
                           s, a);
    return hipGetLastError();
}

// Expert GEMMs take either weight layout; the router's weights are row-major.
template <typename TW, int XM, int NSUB, int EPI, int U = kU, int KW = 1>
hipError_t launch_t(const StreamArgs &a, int n_groups, int zblocks, hipStream_t s) {
    if constexpr (EPI != EPI_LOGITS) {
        if (a.w_frag) return launch_l<TW, XM, NSUB, EPI, U, KW, true>(a, n_groups, zblocks, s);
    }
    return launch_l<TW, XM, NSUB, EPI, U, KW, false>(a, n_groups, zblocks, s);
}

}  // namespace

bool stream_gemm_same_kernel(int dtype, int mode, long est_a, long est_b) {
    // only the fp16 down projection picks its shape from the estimate
    if (dtype != DT_F16 || mode != STREAM_STORE) return true;
    return (est_a >= kStoreWideRows) == (est_b >= kStoreWideRows);
}

hipError_t launch_stream_gemm(const StreamArgs &a, int dtype, int x_dtype, int mode,
                              int n_groups, int zblocks, long est_rows, hipStream_t s) {
    if (n_groups + a.n_sec <= 0 || zblocks <= 0) return hipSuccess;
    if (n_groups + a.n_sec > 65535) return hipErrorInvalidValue;
    if (dtype == DT_F16) {
        // the K-split shapes need K to hold 4 quarters of 4 chunks of 32
        const bool kw_ok = a.K % (a.ksplit * 4 * 4 * 32) == 0;
        if (mode == STREAM_SWIGLU) {
            constexpr int NS = kSwigluNsub, U = kSwigluU, KW = 4;
            if (x_dtype == DT_FP8)
                return kw_ok ? launch_t<f16, DT_FP8, NS, EPI_SWIGLU, kSwigluUFp8, KW>(a, n_groups,
                                                                                    zblocks, s)
                             : launch_t<f16, DT_FP8, 1, EPI_SWIGLU>(a, n_groups, zblocks, s);
            return kw_ok ? launch_t<f16, DT_F16, NS, EPI_SWIGLU, U, KW>(a, n_groups, zblocks, s)
                         : launch_t<f16, DT_F16, 1, EPI_SWIGLU>(a, n_groups, zblocks, s);
        }
        if (mode == STREAM_STORE) {
            if (est_rows >= kStoreWideRows)
                return kw_ok ? launch_t<f16, DT_F16, kStoreNsubWide, EPI_STORE, kStoreUWide, 4>(
                                   a, n_groups, zblocks, s)
                             : launch_t<f16, DT_F16, 2, EPI_STORE>(a, n_groups, zblocks, s);
            return launch_t<f16, DT_F16, 1, EPI_STORE>(a, n_groups, zblocks, s);
        }
        // router: the 4 waves of a block split each K slice and share 64
        // experts, so a block loads its token rows once (not once per wave)
        return kw_ok ? launch_t<f16, DT_F16, 4, EPI_LOGITS, 2, 4>(a, n_groups, zblocks, s)
                     : launch_t<f16, DT_F16, 1, EPI_LOGITS>(a, n_groups, zblocks, s);
    }
    if (mode == STREAM_SWIGLU) return launch_t<float, DT_F32, 1, EPI_SWIGLU>(a, n_groups, zblocks, s);
    if (mode == STREAM_STORE) return launch_t<float, DT_F32, 1, EPI_STORE>(a, n_groups, zblocks, s);
    return launch_t<float, DT_F32, 1, EPI_LOGITS>(a, n_groups, zblocks, s);
}

}  // namespace moe
