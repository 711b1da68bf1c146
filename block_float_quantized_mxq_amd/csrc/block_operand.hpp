// block_operand.hpp -- one lane's share of a bf16 MFMA operand taken from
// block-float weights: the 32 consecutive k of one weight row that start at a
// multiple of 32 (one E8M0 block for MXFP4 / MXFP8, two E4M3 blocks for
// NVFP4), decoded eight at a time into the eight bf16 of a k step.
//
// The MFMA sums over k, so the k order inside a slice may be permuted as long
// as both operands use the same permutation; giving every lane one whole
// block per slice makes its codes one 16-byte (32 for E4M3) load with one
// scale byte.  The decode is exact: every E2M1 value times an E8M0 scale is a
// bf16 (or overflows as it does in fp32), so is every E4M3 value at E8M0 bytes
// of kMx8Lift and above (lower bytes: the split below), and an E2M1 value
// times an E4M3 scale has at most 6 significant bits.
#pragma once

#include "mxq_device.hpp"

namespace mxq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4g_t __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One lane's W codes for one slice: the KE (32, or 16 for E4M3) consecutive k
// of one row starting at a multiple of KE, and their scale byte(s).
template <int FMT, int KE = 32>
struct WFrag {
    static_assert(KE == 32 || (KE == 16 && FMT == kMXFP8), "32 elements, or 16 of E4M3 (16 bytes)");
    static constexpr int DW = (FMT == kMXFP8) ? KE / 4 : 4;
    uint32_t w[DW];
    uint32_t s;  // one E8M0 byte, or two E4M3 bytes (NVFP4) in bits 7:0 and 15:8
};

// NVFP4 rows whose k is an odd multiple of 16 (ROW8): rows are 8-byte aligned,
// so the 16 bytes of a fragment come as two 8-byte loads, and the row's last
// fragment holds one 16-element block: its second half reads as zero codes
// with a unit scale (nothing past the row is read).
typedef uint32_t u32x2g_t __attribute__((ext_vector_type(2)));

template <bool ROW8>
__device__ __forceinline__ void load_fp4_frag16(const uint8_t* crow, const uint8_t* srow, int64_t kb, int64_t k,
                                                uint32_t (&w)[4], uint32_t& s) {
    if constexpr (ROW8) {
        const u32x2g_t* q = reinterpret_cast<const u32x2g_t*>(crow + kb / 2);
        const u32x2g_t a = q[0];
        w[0] = a[0];
        w[1] = a[1];
        if (kb + 32 <= k) {
            const u32x2g_t b = q[1];
            w[2] = b[0];
            w[3] = b[1];
            s = (uint32_t)srow[kb / 16] | ((uint32_t)srow[kb / 16 + 1] << 8);
        } else {
            w[2] = 0u;
            w[3] = 0u;
            s = (uint32_t)srow[kb / 16] | (0x38u << 8);
        }
    } else {
        const u32x4g_t v = *reinterpret_cast<const u32x4g_t*>(crow + kb / 2);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
        s = (uint32_t)srow[kb / 16] | ((uint32_t)srow[kb / 16 + 1] << 8);
    }
}

// Elements past k read as zero codes (with a unit scale).
template <int FMT, int KE, bool ROW8 = false>
__device__ __forceinline__ void load_wfrag(const uint8_t* crow, const uint8_t* srow, int64_t kb, int64_t k,
                                           WFrag<FMT, KE>& f) {
    static_assert(!ROW8 || FMT == kNVFP4, "only NVFP4 rows can be 8-byte multiples");
    if (kb >= k) {
#pragma unroll
        for (int i = 0; i < WFrag<FMT, KE>::DW; ++i) f.w[i] = 0u;
        f.s = FMT == kNVFP4 ? 0x3838u : 127u;
        return;
    }
    if constexpr (FMT == kNVFP4) {
        load_fp4_frag16<ROW8>(crow, srow, kb, k, f.w, f.s);
        return;
    }
    if constexpr (FMT == kMXFP8) {
        const u32x4g_t* q = reinterpret_cast<const u32x4g_t*>(crow + kb);
        const u32x4g_t v0 = q[0];
        f.w[0] = v0[0]; f.w[1] = v0[1]; f.w[2] = v0[2]; f.w[3] = v0[3];
        if constexpr (KE == 32) {
            const u32x4g_t v1 = q[1];
            f.w[4] = v1[0]; f.w[5] = v1[1]; f.w[6] = v1[2]; f.w[7] = v1[3];
        }
        f.s = srow[kb / 32];
    } else {
        const u32x4g_t v = *reinterpret_cast<const u32x4g_t*>(crow + kb / 2);
        f.w[0] = v[0]; f.w[1] = v[1]; f.w[2] = v[2]; f.w[3] = v[3];
        f.s = srow[kb / 32];
    }
}

// The B operand of k step S: the fragment's codes S*8 .. S*8+7 as bf16.
template <int FMT, int S, int KE>
__device__ __forceinline__ bf16x8_t decode_step(const WFrag<FMT, KE>& f) {
    static_assert(S * 8 < KE, "k step inside the fragment");
    uint32_t d[4];
    if constexpr (FMT == kMXFP4) {
        const float se = e8m0_exponent(f.s);
        d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.w[S], se, 0));
        d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.w[S], se, 1));
        d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.w[S], se, 2));
        d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.w[S], se, 3));
    } else if constexpr (FMT == kMXFP8) {
        const float se = e8m0_exponent(f.s);
        d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.w[2 * S], se, false));
        d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.w[2 * S], se, true));
        d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.w[2 * S + 1], se, false));
        d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.w[2 * S + 1], se, true));
    } else {
        // The conversion uses only the exponent of its scale operand, so the
        // E4M3 block scale (16 elements: k steps 0-1, then 2-3) is applied in fp32.
        const float s = e4m3_to_f32(S < 2 ? (f.s & 0xFFu) : ((f.s >> 8) & 0xFFu));
        d[0] = scaled_fp4x2_to_bf16x2<0>(f.w[S], s);
        d[1] = scaled_fp4x2_to_bf16x2<1>(f.w[S], s);
        d[2] = scaled_fp4x2_to_bf16x2<2>(f.w[S], s);
        d[3] = scaled_fp4x2_to_bf16x2<3>(f.w[S], s);
    }
    return __builtin_bit_cast(bf16x8_t, u32x4g_t{d[0], d[1], d[2], d[3]});
}

// MXFP8 fragments whose E8M0 byte is below kMx8Lift (mxq_device.hpp) are not
// exact in bf16.  A wave holding one splits each fragment in two operands:
// the plain part (lifted fragments' codes zeroed) and the lifted part (the
// other fragments' codes zeroed, lifted fragments decoded with byte
// u + kMx8Lift).  The plain part goes into the accumulator as usual; the
// lifted part into a separate sum that is multiplied by 2^-kMx8Lift in fp32.
template <int FMT, int KE>
__device__ __forceinline__ bool frag_lifted(const WFrag<FMT, KE>& f) {
    return mx_lifted<FMT>(f.s);
}

template <int FMT, int S, bool LIFTED, int KE>
__device__ __forceinline__ bf16x8_t decode_step_part(const WFrag<FMT, KE>& f) {
    static_assert(FMT == kMXFP8, "only MXFP8 fragments are lifted");
    const bool lo = frag_lifted(f);
    const bool keep = LIFTED ? lo : !lo;
    WFrag<FMT, KE> g;
#pragma unroll
    for (int d = 0; d < WFrag<FMT, KE>::DW; ++d) g.w[d] = keep ? f.w[d] : 0u;
    g.s = LIFTED ? (lo ? f.s + kMx8Lift : 127u) : f.s;
    return decode_step<FMT, S>(g);
}

}  // namespace mxq
