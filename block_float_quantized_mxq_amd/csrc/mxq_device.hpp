// mxq_device.hpp -- device-side building blocks shared by the libmxq kernels:
// in-register decode of E2M1 / E4M3 codes and E8M0 / E4M3 block scales, the
// bf16 dot product, and wave64 cross-lane sums.
//
// Decode follows the "Decoding block-float formats in software" section of the
// "MLxcel 0.8 release" post (and slide 12 of the Strix Halo talk): codes are
// turned into 16-bit floats inside the kernel, exactly, and then multiplied
// with the activations.  On gfx950 the conversion is one hardware instruction
// per two codes (V_CVT_SCALEF32_PK_BF16_FP4 / _FP8), which replaces the pages'
// bit-placement trick: every E2M1 and every finite E4M3 value is exactly
// representable in bf16.  An E8M0 block scale is a power of two and goes into
// the conversion's scale operand; an E4M3 block scale (NVFP4) has mantissa
// bits, which that operand ignores, so it multiplies the block's fp32 partial
// sum instead.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.hpp"

namespace mxq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Elements per scale block.
template <int FMT> struct BlockSize { static constexpr int value = (FMT == kNVFP4) ? 16 : 32; };


// ---- code decode: packed codes -> bf16 pairs (element 2j in the low half) ----

// Byte `SEL` of `w` holds two E2M1 codes (even element in bits 3:0).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// Half-word `HI` of `w` holds two E4M3 codes (even element in the low byte).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Decode DW code dwords into bf16 pairs: 4 pairs per dword for E2M1, 2 for E4M3.
template <int FMT, int DW>
__device__ __forceinline__ void decode_dwords(const uint32_t (&c)[DW], uint32_t (&p)[(FMT == kMXFP8) ? 2 * DW : 4 * DW]) {
#pragma unroll
    for (int d = 0; d < DW; ++d) {
        if constexpr (FMT == kMXFP8) {
            p[2 * d + 0] = fp8x2_to_bf16x2<false>(c[d]);
            p[2 * d + 1] = fp8x2_to_bf16x2<true>(c[d]);
        } else {
            p[4 * d + 0] = fp4x2_to_bf16x2<0>(c[d]);
            p[4 * d + 1] = fp4x2_to_bf16x2<1>(c[d]);
            p[4 * d + 2] = fp4x2_to_bf16x2<2>(c[d]);
            p[4 * d + 3] = fp4x2_to_bf16x2<3>(c[d]);
        }
    }
}

// Same with an E8M0 block scale applied by the conversion: `sexp` is an fp32
// whose exponent field is the E8M0 byte (the conversion uses only the
// exponent of its scale operand, so byte 0 means 2^-127 and byte 255 gives
// NaN, as the format defines).  Each result is q * 2^(u-127) rounded to bf16:
// exact for every E2M1 code at every byte, and for every E4M3 code at bytes
// of kMx8Lift and above (see below).
template <int FMT, int DW>
__device__ __forceinline__ void decode_dwords_scaled(const uint32_t (&c)[DW], float sexp,
                                                     uint32_t (&p)[(FMT == kMXFP8) ? 2 * DW : 4 * DW]) {
#pragma unroll
    for (int d = 0; d < DW; ++d) {
        if constexpr (FMT == kMXFP8) {
            p[2 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[d], sexp, false));
            p[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[d], sexp, true));
        } else {
            p[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], sexp, 0));
            p[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], sexp, 1));
            p[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], sexp, 2));
            p[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], sexp, 3));
        }
    }
}

// E8M0 byte as the exponent field of an fp32 (the scale operand above).
__device__ __forceinline__ float e8m0_exponent(uint32_t u) { return __builtin_bit_cast(float, (u & 0xFFu) << 23); }

// Exactness of the scaled conversion, measured on gfx950 over every code and
// every E8M0 byte: the result is q * 2^(u-127) rounded to nearest even in bf16,
// with bf16 subnormals, overflow to infinity and NaN for byte 255 (whatever the
// code).  An E2M1 value has at most two significant bits and is at least 2^-1,
// so every MXFP4 result is a bf16 (or overflows in fp32 just the same).  An
// E4M3 value keeps four significant bits down to 2^-9, so q * 2^(u-127) needs
// bits down to 2^(u-136), finer than bf16's smallest subnormal step 2^-133
// when u < 3.  MXFP8 blocks with such a byte are "lifted": decoded with byte
// u + kMx8Lift (exact) and their fp32 contribution multiplied by
// 2^-kMx8Lift, which restores q * 2^(u-127) exactly in fp32.
constexpr uint32_t kMx8Lift = 3;
constexpr float kMx8Unlift = 0.125f;  // 2^-kMx8Lift
template <int FMT>
__device__ __forceinline__ bool mx_lifted(uint32_t u) { return FMT == kMXFP8 && u < kMx8Lift; }

// Two E2M1 codes (byte SEL of w) times an fp32 scale s (an E4M3 block scale),
// as a bf16 pair: q * s has at most 6 significant bits, so the bf16 is exact.
template <int SEL>
__device__ __forceinline__ uint32_t scaled_fp4x2_to_bf16x2(uint32_t w, float s) {
    const f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    const bf16x2_t b = {(__bf16)(f[0] * s), (__bf16)(f[1] * s)};
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t p) { return __builtin_bit_cast(float, p & 0xFFFF0000u); }

// ---- block scales -------------------------------------------------------------

// E8M0 byte u -> 2^(u-127) as fp32 (u = 0 gives the subnormal 2^-127); 0xFF -> NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t u) {
    float v = __builtin_amdgcn_ldexpf(1.0f, (int)u - 127);
    return (u == 255u) ? __builtin_nanf("") : v;
}

// E4M3 (OCP) byte -> fp32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// ---- synchronisation ---------------------------------------------------------------

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations
// only, so global loads that are still in flight are not drained (a plain
// __syncthreads() waits for them too).  The asm is a compiler memory barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---- arithmetic -------------------------------------------------------------------

// c + a.lo*b.lo + a.hi*b.hi with bf16 inputs and fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// SwiGLU activation a = bf16(silu(g) * u) with silu(g) = g / (1 + e^-g), in
// fp32, the product rounded to the nearest bf16 (ties to even).  Below
// g = -64, 1 + e^-g equals e^-g far beyond fp32 precision (e^-64 < 2^-92),
// and from g = -88.7 e^-g overflows (the quotient would become 0 while
// silu(g) is still a normal fp32 number), so there silu(g) = g e^g is formed
// as (g e^(g/2)) e^(g/2): g/2 is exact, both factors stay normal down to
// g = -174, and the result is within a few ulp (zero below that, as it is
// in fp32).
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u) {
    float s;
    if (g >= -64.0f) {
        s = g / (1.0f + expf(-g));
    } else {
        const float e = expf(0.5f * g);
        s = g * e * e;
    }
    return __builtin_bit_cast(uint16_t, (__bf16)(s * u));
}

// DPP controls (GFX9 encoding).
enum : int { kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140 };

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G in {1,2,4,8,16,32,64}); every lane of a
// group ends with the group total.  The order of additions is fixed.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += dpp_f32<kDppQuadXor1>(v);
    if constexpr (G >= 4) v += dpp_f32<kDppQuadXor2>(v);
    if constexpr (G >= 8) v += dpp_f32<kDppRowHalfMirror>(v);
    if constexpr (G >= 16) v += dpp_f32<kDppRowMirror>(v);
    if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

}  // namespace mxq
