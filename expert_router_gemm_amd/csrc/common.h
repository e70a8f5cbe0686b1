// common.h -- device helpers shared by the libmoe kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// dtype codes, identical to moe_dtype in include/moe.h
enum : int { DT_F32 = 0, DT_F16 = 1, DT_FP8 = 2 };

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- MFMA
// 16x16 output tile, fp32 accumulators.  Lane l holds C[4*(l/16) + j][l%16]
// for j = 0..3 (same layout for both instructions below).
//
// f16: v_mfma_f32_16x16x32_f16.  Lane l supplies A[l%16][8*(l/16) + 0..7]
// and B[8*(l/16) + 0..7][l%16].
__device__ __forceinline__ f32x4 mfma16(const f16x8 &a, const f16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// f32: four v_mfma_f32_16x16x4_f32, one per element of the lane's 4-vector.
// Lane l supplies A[l%16][4*(l/16) + j] and B[4*(l/16) + j][l%16] in step j.
__device__ __forceinline__ f32x4 mfma16(const f32x4 &a, const f32x4 &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

// Elements per 16-byte lane fragment, and the K span one fragment-wide MFMA
// step covers (4 lane groups of 16 lanes).
template <typename T> struct Frag;
template <> struct Frag<f16> {
    typedef f16x8 vec;
    static constexpr int kElems = 8;
};
template <> struct Frag<float> {
    typedef f32x4 vec;
    static constexpr int kElems = 4;
};

template <typename T>
__device__ __forceinline__ typename Frag<T>::vec load16(const T *p) {
    return *reinterpret_cast<const typename Frag<T>::vec *>(p);
}

// OCP E4M3 code -> the same value times 2^-8 as an fp16 bit pattern: moving
// the sign to bit 15 and the 7 exponent/mantissa bits to bits 13..7 keeps the
// mantissa and rebiases the exponent from 7 to 15 (a factor 2^-8), and an
// E4M3 subnormal m*2^-9 lands on the fp16 subnormal m*2^-17.  Exact for every
// finite code; the 2^8 is folded into the row scale.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2_bits(uint32_t two) {
    // two = c0 | c1 << 8
    uint32_t lo = ((two & 0x7fu) << 7) | ((two & 0x80u) << 8);
    uint32_t hi = ((two & 0x7f00u) << 15) | ((two & 0x8000u) << 16);
    return lo | hi;
}

__device__ __forceinline__ f16x8 e4m3x8_to_f16x8_scaled(u32x2 codes) {
    u32x4 r;
    r[0] = e4m3x2_to_f16x2_bits(codes[0] & 0xffffu);
    r[1] = e4m3x2_to_f16x2_bits(codes[0] >> 16);
    r[2] = e4m3x2_to_f16x2_bits(codes[1] & 0xffffu);
    r[3] = e4m3x2_to_f16x2_bits(codes[1] >> 16);
    return __builtin_bit_cast(f16x8, r);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float siluf_(float z) { return z / (1.0f + expf(-z)); }

// Round-to-nearest-even conversions for outputs.
__device__ __forceinline__ f16 to_f16(float v) { return (f16)v; }
// The same for 8 fp32 values, two per v_cvt_pk_f16_f32 (round to nearest
// even).  Written as the instruction itself so the compiler cannot fold the
// conversion into the fma that produced a value (v_fma_mixlo_f16 rounds
// the exact result once, to fp16), which it does in some contexts and not
// in others: the combine's two code paths must round alike (the separate
// combine kernel's 8-wide vector conversion compiles to this instruction).
typedef float f32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 to_f16x8_of_f32(f32x8 v) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r[j]) : "v"(v[2 * j]), "v"(v[2 * j + 1]));
    return __builtin_bit_cast(f16x8, r);
}

}  // namespace moe
