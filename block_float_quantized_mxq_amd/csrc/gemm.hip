// gemm.hip -- prefill GEMM on block-float weights: Y[m][i] = sum_k X[m][k] * W[i][k].
//
// Prefill is compute bound ("The memory wall" section of the "MLxcel 0.8
// release" post, slide 15 of the talk); the pages' fast path decodes the
// quantized weights on the GPU and feeds the matrix unit ("Decoding block-float
// formats in software", slide 12).  Here each workgroup owns a BM x BN output
// tile; per BK slice it stages X into LDS, decodes the W slice to bf16 (block
// scale folded into the conversion: exact for normal-range weights) into LDS,
// and runs bf16 MFMA 32x32x16 with fp32 accumulation.  The NVFP4 per-tensor
// scale multiplies the fp32 result; the bf16 output is rounded to nearest even
// from that fp32 value.
#include "kernels.hpp"
#include "mxq_device.hpp"

namespace mxq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4g_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row (padding breaks bank conflicts)
constexpr int kGemmThreads = 256;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two E2M1 codes (byte SEL of w) times an arbitrary fp32 scale s, as a bf16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t scaled_fp4x2_to_bf16x2(uint32_t w, float s) {
    const f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    const bf16x2_t b = {(__bf16)(f[0] * s), (__bf16)(f[1] * s)};
    return __builtin_bit_cast(uint32_t, b);
}

// Decode 32 consecutive elements of one weight row, starting at element k0,
// to bf16 (scale folded in) into 16 dwords.  Elements past k are zero.
template <int FMT>
__device__ __forceinline__ void decode_w32(const uint8_t* crow, const uint8_t* srow, int64_t k0, int64_t k,
                                           uint32_t (&out)[16]) {
    if (k0 >= k) {
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = 0u;
        return;
    }
    if constexpr (FMT == kMXFP8) {
        const u32x4g_t* p = reinterpret_cast<const u32x4g_t*>(crow + k0);
        const u32x4g_t v0 = p[0], v1 = p[1];
        const float s = e8m0_to_f32(srow[k0 / 32]);
        const uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            out[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], s, false));
            out[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], s, true));
        }
    } else {
        const u32x4g_t v = *reinterpret_cast<const u32x4g_t*>(crow + k0 / 2);
        const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
        if constexpr (FMT == kMXFP4) {
            // E8M0 scales are powers of two: the conversion applies them exactly.
            const float s = e8m0_to_f32(srow[k0 / 32]);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                out[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 0));
                out[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 1));
                out[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 2));
                out[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 3));
            }
        } else {
            // The conversion instruction uses only the exponent of its scale operand,
            // so E4M3 block scales (which carry mantissa bits) are applied in fp32:
            // q * s has at most 6 significant bits, so the bf16 result is exact.
            const float s0 = e4m3_to_f32(srow[k0 / 16]);
            const float s1 = e4m3_to_f32(srow[k0 / 16 + 1]);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const float s = d < 2 ? s0 : s1;
                out[4 * d + 0] = scaled_fp4x2_to_bf16x2<0>(w[d], s);
                out[4 * d + 1] = scaled_fp4x2_to_bf16x2<1>(w[d], s);
                out[4 * d + 2] = scaled_fp4x2_to_bf16x2<2>(w[d], s);
                out[4 * d + 3] = scaled_fp4x2_to_bf16x2<3>(w[d], s);
            }
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gscale,
                                                            const uint16_t* __restrict__ x, void* __restrict__ yv,
                                                            int y_bf16, int64_t m, int64_t n, int64_t k) {
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;

    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t sbytes = k / block_elems(FMT);

    // Loader mapping: thread -> (tile row tid/2, 32-element half tid%2).
    const int lr = tid >> 1, lh = tid & 1;
    int64_t xr = m0 + lr;
    xr = xr < m ? xr : m - 1;
    int64_t wr = n0 + lr;
    wr = wr < n ? wr : n - 1;
    const uint16_t* xrow = x + xr * k;
    const uint8_t* crow = codes + wr * rowbytes;
    const uint8_t* srow = scales + wr * sbytes;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    for (int64_t kt = 0; kt < k; kt += kBK) {
        const int64_t ka = kt + lh * 32;
        uint32_t xa[16];
        if (ka < k) {
            const u32x4g_t* p = reinterpret_cast<const u32x4g_t*>(xrow + ka);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4g_t v = p[q];
                xa[4 * q] = v[0]; xa[4 * q + 1] = v[1]; xa[4 * q + 2] = v[2]; xa[4 * q + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) xa[q] = 0u;
        }
        uint32_t wb[16];
        decode_w32<FMT>(crow, srow, ka, k, wb);

        __syncthreads();  // previous slice fully consumed
        u32x4g_t* ad = reinterpret_cast<u32x4g_t*>(As + lr * kLdsStride + lh * 32);
        u32x4g_t* bd = reinterpret_cast<u32x4g_t*>(Bs + lr * kLdsStride + lh * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ad[q] = u32x4g_t{xa[4 * q], xa[4 * q + 1], xa[4 * q + 2], xa[4 * q + 3]};
            bd[q] = u32x4g_t{wb[4 * q], wb[4 * q + 1], wb[4 * q + 2], wb[4 * q + 3]};
        }
        __syncthreads();

#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kk = ks * 16 + (lane >> 5) * 8;
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ar = wm * 64 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8_t*>(As + ar * kLdsStride + kk);
                const int br = wn * 64 + i * 32 + (lane & 31);
                bfr[i] = *reinterpret_cast<const bf16x8_t*>(Bs + br * kLdsStride + kk);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    const float g = (FMT == kNVFP4) ? gscale[0] : 1.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
                if (row >= m) continue;
                const float v = acc[i][j][e] * g;
                if (y_bf16) reinterpret_cast<uint16_t*>(yv)[row * n + col] = f32_to_bf16_rne(v);
                else reinterpret_cast<float*>(yv)[row * n + col] = v;
            }
        }
}

template <int FMT>
static void launch_gemm_inst(const GemmArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.n + kBN - 1) / kBN), (unsigned)((a.m + kBM - 1) / kBM));
    hipLaunchKernelGGL((gemm_kernel<FMT>), grid, dim3(kGemmThreads), 0, st, a.codes, a.scales, a.gscale, a.x, a.y,
                       a.y_bf16, a.m, a.n, a.k);
}

bool launch_gemm(const GemmArgs& a, hipStream_t st) {
    switch (a.fmt) {
        case kMXFP4: launch_gemm_inst<kMXFP4>(a, st); return true;
        case kMXFP8: launch_gemm_inst<kMXFP8>(a, st); return true;
        case kNVFP4: launch_gemm_inst<kNVFP4>(a, st); return true;
    }
    return false;
}

}  // namespace mxq
