// quantize.hip -- block-float quantizer: bf16 rows -> MXFP4 / MXFP8 / NVFP4
// codes and block scales (the inverse of the decode the other kernels run).
//
// The ROCm status table of the "Build from source" manual (section "Current
// status", row "mxfp8, mxfp4 checkpoints") requantizes vendor FP8 block
// checkpoints to MXFP8 when a model is loaded.  The conversion follows OCP MX
// v1.0: shared exponent floor(log2 amax) - emax (emax 2 for E2M1, 8 for
// E4M3), clamped to [-127, 127], zero blocks at -127; NVFP4 takes the E4M3
// block scale of amax / (6 g) for the caller's per-tensor scale g.  Elements
// are rounded to the nearest value of the element format, ties to the even
// code, saturating at its largest value; the input's sign is kept.
//
// One lane per block: it loads the block's bf16 values (64 or 32 bytes),
// finds the maximum magnitude, picks the scale and writes the codes (16, 32 or
// 8 bytes) and the scale byte.  Every step is an exact power-of-two scaling or
// a round-to-nearest-even in fp32, plus, for NVFP4, two correctly rounded fp32
// divisions; HBM bound (2 bytes read per element).
#include "kernels.hpp"
#include "mxq_device.hpp"
#include "rows_core.hpp"

namespace mxq {

// |p| rounded to the grid of mbits mantissa bits and minimum exponent emin,
// saturating at maxv (a >= 0).
__device__ __forceinline__ float quant_mag(float a, int mbits, int emin, float maxv) {
    if (a == 0.0f) return 0.0f;
    if (a >= maxv) return maxv;
    int e = __builtin_amdgcn_frexp_expf(a) - 1;  // floor(log2 a)
    e = e < emin ? emin : e;
    const float r = __builtin_rintf(__builtin_amdgcn_ldexpf(a, mbits - e));  // ties to even
    const float v = __builtin_amdgcn_ldexpf(r, e - mbits);
    return v > maxv ? maxv : v;
}

__device__ __forceinline__ uint32_t e4m3_code(float r) {  // r a representable E4M3 magnitude
    if (r < 0.015625f) return (uint32_t)(r * 512.0f);     // subnormal: multiples of 2^-9
    const int e = __builtin_amdgcn_frexp_expf(r) - 1;
    const uint32_t m = (uint32_t)(__builtin_amdgcn_ldexpf(r, -e) * 8.0f) - 8u;
    return ((uint32_t)(e + 7) << 3) | m;
}

// 32 fp32 quotients -> E4M3 codes (8 dwords, element j in byte j % 4 of
// dword j / 4): the hardware conversion with a unit scale operand, the
// quotients first clamped to +-448.  The conversion does not saturate the way
// the definition does (quotients reach 512); the rest -- nearest value, ties
// to the even code, subnormals, signed zeros -- matches it bit for bit.
__device__ __forceinline__ void e4m3_block_codes(const float (&p)[32], uint32_t (&out)[8]) {
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
        const float p0 = __builtin_fminf(__builtin_fmaxf(p[j], -448.0f), 448.0f);
        const float p1 = __builtin_fminf(__builtin_fmaxf(p[j + 1], -448.0f), 448.0f);
        const s16x2_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2_t{0, 0}, p0, p1, 1.0f, false);
        out[j / 4] |= ((uint32_t)(uint16_t)hw[0]) << (8 * (j % 4));
    }
}

// OCP MX shared exponent of a block of E4M3 elements with largest magnitude
// amax: floor(log2 amax) - 8, clamped to [-127, 127]; -127 for a zero block.
__device__ __forceinline__ int mx8_shared_exponent(float amax) {
    int se = -127;
    if (amax > 0.0f) {
        se = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
        se = se < -127 ? -127 : (se > 127 ? 127 : se);
    }
    return se;
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ gscale,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                       int64_t rows, int64_t k) {
    constexpr int BS = BlockSize<FMT>::value;
    const int64_t nb = k / BS;
    // grid-stride loop: the dispatch's work-item count is a 32-bit number
    for (int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x; blk < rows * nb; blk += (int64_t)gridDim.x * 256) {
    const int64_t r = blk / nb, b = blk % nb;

    uint32_t w[BS / 2];  // bf16 pairs
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + r * k + b * BS);
#pragma unroll
    for (int i = 0; i < BS / 8; ++i) {
        const u32x4_t v = src[i];
        w[4 * i + 0] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < BS / 2; ++i) {
        const float lo = __builtin_fabsf(bf16_lo_to_f32(w[i])), hi = __builtin_fabsf(bf16_hi_to_f32(w[i]));
        amax = lo > amax ? lo : amax;
        amax = hi > amax ? hi : amax;
    }

    // p = v * mul (MX: mul = 2^-se, exact) or p = v / den (NVFP4)
    float mul = 1.0f, den = 1.0f;
    bool zero = false;
    if constexpr (FMT == kNVFP4) {
        const float g = gscale[0];
        const float t = amax / (6.0f * g);
        const float s = quant_mag(t, 3, -6, 448.0f);
        scales[blk] = (uint8_t)e4m3_code(s);
        zero = s == 0.0f;
        den = s * g;
    } else {
        constexpr int emax = FMT == kMXFP4 ? 2 : 8;
        int se = -127;
        if (amax > 0.0f) {
            se = __builtin_amdgcn_frexp_expf(amax) - 1 - emax;
            se = se < -127 ? -127 : (se > 127 ? 127 : se);
        }
        scales[blk] = (uint8_t)(se + 127);
        mul = __builtin_amdgcn_ldexpf(1.0f, -se);  // se >= -127: 2^127 at most, normal
    }

    uint32_t out[FMT == kMXFP8 ? BS / 4 : BS / 8] = {};
    if constexpr (FMT == kMXFP8) {
        float p[BS];
#pragma unroll
        for (int j = 0; j < BS; ++j) p[j] = ((j & 1) ? bf16_hi_to_f32(w[j / 2]) : bf16_lo_to_f32(w[j / 2])) * mul;
        e4m3_block_codes(p, out);
    } else {
        // E2M1 codes by the hardware conversion with a unit scale operand: it
        // rounds to nearest with ties to even, saturates and keeps the sign,
        // as the definition does (checked bit for bit against the oracle on
        // ties, saturating quotients and signed zeros)
        float p[BS];
        if constexpr (FMT == kNVFP4) {
            // p = RN(v / den).  One correctly rounded reciprocal y = RN(1/den)
            // per block, then per element q0 = RN(v y) and the residual step
            // RN(q0 + (v - q0 den) y) (Markstein's correction, both by fma):
            // that is the correctly rounded quotient whenever every
            // intermediate stays a normal number, which the exponent bounds
            // below guarantee (verified exhaustively for every fp32 den and
            // bf16 v mantissa).  Other operands, zeros among them, take the
            // division itself.
            const bool blk_fast = !zero && den >= 0x1p-40f && den <= 0x1p40f;
            const float y = blk_fast ? 1.0f / den : 1.0f;
            bool slow = false;
#pragma unroll
            for (int j = 0; j < BS; ++j) {
                const float v = (j & 1) ? bf16_hi_to_f32(w[j / 2]) : bf16_lo_to_f32(w[j / 2]);
                const float a = __builtin_fabsf(v);
                const bool fast = blk_fast && a >= 0x1p-30f && a <= 0x1p80f;
                const float q0 = __fmul_rn(v, y);
                const float rsd = __builtin_fmaf(-q0, den, v);
                p[j] = __builtin_fmaf(rsd, y, q0);
                slow |= !fast;
            }
            if (slow) {
#pragma unroll
                for (int j = 0; j < BS; ++j) {
                    const float v = (j & 1) ? bf16_hi_to_f32(w[j / 2]) : bf16_lo_to_f32(w[j / 2]);
                    const float a = __builtin_fabsf(v);
                    const bool fast = blk_fast && a >= 0x1p-30f && a <= 0x1p80f;
                    if (!fast) p[j] = zero ? __builtin_copysignf(0.0f, v) : v / den;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < BS; ++j) p[j] = ((j & 1) ? bf16_hi_to_f32(w[j / 2]) : bf16_lo_to_f32(w[j / 2])) * mul;
        }
#pragma unroll
        for (int j = 0; j < BS; j += 2) {
            const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p[j], p[j + 1], 1.0f, 0);
            out[j / 8] |= (c & 0xFFu) << (4 * (j % 8));
        }
    }
    if constexpr (FMT == kMXFP8) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + r * k + b * BS);
        dst[0] = u32x4_t{out[0], out[1], out[2], out[3]};
        dst[1] = u32x4_t{out[4], out[5], out[6], out[7]};
    } else if constexpr (FMT == kMXFP4) {
        *reinterpret_cast<u32x4_t*>(codes + r * (k / 2) + b * 16) = u32x4_t{out[0], out[1], out[2], out[3]};
    } else {
        *reinterpret_cast<u32x2_t*>(codes + r * (k / 2) + b * 8) = u32x2_t{out[0], out[1]};
    }
    }
}

// Workgroups of a block-per-lane launch over nb blocks: one lane per block up
// to 2^20 workgroups, beyond that the kernels' grid-stride loops take over.
static dim3 block_grid(int64_t nb) {
    const int64_t wg = (nb + 255) / 256;
    return dim3((unsigned)(wg < (int64_t(1) << 20) ? wg : (int64_t(1) << 20)));
}

bool launch_quantize(const QuantizeArgs& a, hipStream_t st) {
    const int64_t nb = a.rows * (a.k / block_elems(a.fmt));
    const dim3 grid = block_grid(nb), block(256);
    switch (a.fmt) {
        case kMXFP4: hipLaunchKernelGGL(quantize_kernel<kMXFP4>, grid, block, 0, st, a.x, a.gscale, a.codes, a.scales, a.rows, a.k); return true;
        case kMXFP8: hipLaunchKernelGGL(quantize_kernel<kMXFP8>, grid, block, 0, st, a.x, a.gscale, a.codes, a.scales, a.rows, a.k); return true;
        case kNVFP4: hipLaunchKernelGGL(quantize_kernel<kNVFP4>, grid, block, 0, st, a.x, a.gscale, a.codes, a.scales, a.rows, a.k); return true;
    }
    return false;
}

// ---- FP8 block checkpoint -> MXFP8 ------------------------------------------------
//
// The ROCm status table of the "Build from source" manual (section "Current
// status", row "mxfp8, mxfp4 checkpoints") converts vendor FP8 checkpoints --
// E4M3 codes with one fp32 scale per 128 x 128 tile -- to MXFP8 when a model
// loads.  Each lane takes one 32-element block of a row: v = fl32(E4M3(c) * s)
// with the block's tile scale s (the block lies in one tile: bk % 32 == 0),
// then the OCP MX conversion above.  Reads 1 byte and writes 1 + 1/32 bytes
// per element: HBM bound.
__global__ __launch_bounds__(256) void requant_fp8_kernel(const uint8_t* __restrict__ codes_in,
                                                          const float* __restrict__ tile_scales,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                          int64_t n, int64_t k, int64_t bn, int64_t bk) {
    const int64_t nb = k / 32;
    const int64_t tcols = (k + bk - 1) / bk;
    for (int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x; blk < n * nb; blk += (int64_t)gridDim.x * 256) {
        const int64_t r = blk / nb, b = blk % nb;
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(codes_in + r * k + b * 32);
        const u32x4_t c0 = __builtin_nontemporal_load(src), c1 = __builtin_nontemporal_load(src + 1);
        const uint32_t cw[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const float s = tile_scales[(r / bn) * tcols + (b * 32) / bk];
        float v[32];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            v[j] = e4m3_to_f32((cw[j / 4] >> (8 * (j % 4))) & 0xFFu) * s;  // exact decode, one fp32 rounding
            const float a = __builtin_fabsf(v[j]);
            amax = a > amax ? a : amax;
        }
        const int se = mx8_shared_exponent(amax);
        scales[blk] = (uint8_t)(se + 127);
        // exact scaling (|v * mul| < 512); a product below fp32's normal range
        // lies far below E4M3's smallest step and rounds to a signed zero either way
        const float mul = __builtin_amdgcn_ldexpf(1.0f, -se);
        float p[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) p[j] = v[j] * mul;
        uint32_t out[8] = {};
        e4m3_block_codes(p, out);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + r * k + b * 32);
        dst[0] = u32x4_t{out[0], out[1], out[2], out[3]};
        dst[1] = u32x4_t{out[4], out[5], out[6], out[7]};
    }
}

bool launch_requant_fp8(const RequantArgs& a, hipStream_t st) {
    const int64_t nb = a.n * (a.k / 32);
    hipLaunchKernelGGL(requant_fp8_kernel, block_grid(nb), dim3(256), 0, st, a.codes_in, a.tile_scales, a.codes,
                       a.scales, a.n, a.k, a.bn, a.bk);
    return true;
}

}  // namespace mxq
