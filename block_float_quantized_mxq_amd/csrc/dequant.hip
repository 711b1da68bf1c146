// dequant.hip -- decode-only kernel: block-float weights to fp32, using the
// same register decode as the GEMV, MoE and GEMM kernels, so that the decode
// can be checked bit for bit.
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

// One thread per code chunk: w[r][j] = fl32(q * 2^(u-127)) (MX) or
// fl32((q * s) * g) (NVFP4), using the same register decode as the GEMV.
template <int FMT, int CB>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ gscale, float* __restrict__ w,
                                                           int64_t rows, int64_t k) {
    using CS = ChunkShape<FMT, CB>;
    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t nchunks = rowbytes / CB;
    const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (id >= rows * nchunks) return;
    const int64_t r = id / nchunks, c = id % nchunks;
    const uint8_t* srow = scales + r * (k / CS::BS);
    uint32_t cw[CS::DW];
    load_code_chunk<CB>(codes + r * rowbytes + c * CB, cw);
    uint32_t wp[CS::NP];
    decode_dwords<FMT, CS::DW>(cw, wp);
    float* out = w + r * k + c * CS::KPC;
    const float g = (FMT == kNVFP4) ? gscale[0] : 1.0f;
#pragma unroll
    for (int t = 0; t < CS::NP; ++t) {
        const int64_t e = c * CS::KPC + 2 * t;  // element index within the row
        float s;
        if constexpr (FMT == kNVFP4) s = e4m3_to_f32(srow[e / 16]);
        else s = e8m0_to_f32(srow[e / 32]);
        float lo = bf16_lo_to_f32(wp[t]) * s;
        float hi = bf16_hi_to_f32(wp[t]) * s;
        if constexpr (FMT == kNVFP4) {
            lo *= g;
            hi *= g;
        }
        out[2 * t] = lo;
        out[2 * t + 1] = hi;
    }
}

template <int FMT, int CB>
static void launch_dequant_inst(const DequantArgs& a, hipStream_t st) {
    const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
    const int64_t total = a.rows * nchunks;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((dequant_kernel<FMT, CB>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a.codes, a.scales,
                       a.gscale, a.w, a.rows, a.k);
}

bool launch_dequant(const DequantArgs& a, hipStream_t st) {
    const bool wide = (code_bytes_per_row(a.fmt, a.k) % 16) == 0;
    switch (a.fmt) {
        case kMXFP4: launch_dequant_inst<kMXFP4, 16>(a, st); return true;
        case kMXFP8: launch_dequant_inst<kMXFP8, 16>(a, st); return true;
        case kNVFP4:
            if (wide) launch_dequant_inst<kNVFP4, 16>(a, st);
            else launch_dequant_inst<kNVFP4, 8>(a, st);
            return true;
    }
    return false;
}

}  // namespace mxq
