// dequant.hip -- decode-only kernel: block-float weights to fp32 through the
// very decode the GEMV, MoE and GEMM kernels run, so that the decode can be
// checked bit for bit against the format definitions.
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

// One thread per code chunk.  MX formats: the codes go through the scaled
// conversion with the block's E8M0 byte in its scale operand (bf16 out), as
// in every product kernel; MXFP8 blocks with a byte below kMx8Lift are
// decoded with byte u + kMx8Lift and multiplied by 2^-kMx8Lift in fp32, as
// the product kernels scale their partial sums.  NVFP4: unit-scale decode,
// times the E4M3 block scale in fp32 (exact: q * s has at most 6 significant
// bits), times the per-tensor scale g.  The result is w = fl32(q * 2^(u-127))
// or fl32((q * s) * g) for every code and every scale byte.
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
    uint32_t sb[CS::NSG];
    load_scale_bytes<FMT, CB>(srow, c, sb);
    uint32_t wp[CS::NP];
    float mul[CS::NSG];
    if constexpr (FMT == kNVFP4) {
        decode_dwords<FMT, CS::DW>(cw, wp);
#pragma unroll
        for (int q = 0; q < CS::NSG; ++q) mul[q] = e4m3_to_f32(sb[q]);
    } else {
        const uint32_t u = sb[0];
        const bool lo = mx_lifted<FMT>(u);
        decode_dwords_scaled<FMT, CS::DW>(cw, e8m0_exponent(lo ? u + kMx8Lift : u), wp);
        mul[0] = lo ? kMx8Unlift : 1.0f;
    }
    float* out = w + r * k + c * CS::KPC;
    const float g = (FMT == kNVFP4) ? gscale[0] : 1.0f;
#pragma unroll
    for (int t = 0; t < CS::NP; ++t) {
        const float m = mul[t / CS::PPS];
        float lo = bf16_lo_to_f32(wp[t]) * m;
        float hi = bf16_hi_to_f32(wp[t]) * m;
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
