// gemv.hip -- dense block-float GEMV (decode projection) and the decode-only
// dequant kernel.
//
// y[b][i] = sum_k W[i][k] * x[b][k]: the quantized matrix-vector product that
// the "Profiling set the porting order" section of the "MLxcel 0.8 release"
// post measures at 95% of dense decode GPU time.  It reads every weight byte
// once, so it is bound by HBM bandwidth; the kernel streams rows with 128-bit
// loads (rows_core.hpp) and does all arithmetic in registers.
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

template <int FMT, int CB, int B, int G, int S, int R>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        const float* __restrict__ gscale,
                                                        const uint16_t* __restrict__ x, float* __restrict__ y,
                                                        int64_t n, int64_t k, int batch) {
    using T = RowTile<G, S, R>;
    __shared__ float red[S > 1 ? S * T::ROWSETS * R * B : 1];
    const uint16_t* xs[B];
    float* ys[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        xs[b] = x + (int64_t)(b < batch ? b : 0) * k;
        ys[b] = b < batch ? y + (int64_t)b * n : nullptr;
    }
    const float gmul = (FMT == kNVFP4) ? gscale[0] : 1.0f;
    const int64_t row0 = (int64_t)blockIdx.x * T::ROWS;
    rows_core<FMT, CB, B, G, S, R>(codes, scales, n, k, row0, xs, ys, gmul, red);
}

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

// ---- launchers -------------------------------------------------------------------------

template <int FMT, int CB, int B, int G, int S, int R>
static void launch_gemv_inst(const GemvArgs& a, hipStream_t st) {
    using T = RowTile<G, S, R>;
    const int64_t blocks = (a.n + T::ROWS - 1) / T::ROWS;
    hipLaunchKernelGGL((gemv_kernel<FMT, CB, B, G, S, R>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a.codes,
                       a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch);
}

template <int FMT, int CB, int B>
static bool launch_gemv_b(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
#define MXQ_GEMV_CASE(G_, S_, R_)                                   \
    if (cfg.g == G_ && cfg.s == S_ && cfg.r == R_) {               \
        launch_gemv_inst<FMT, CB, B, G_, S_, R_>(a, st);           \
        return true;                                              \
    }
    MXQ_GEMV_CONFIGS(MXQ_GEMV_CASE)
#undef MXQ_GEMV_CASE
    return false;
}

template <int FMT, int CB>
static bool launch_gemv_cb(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    if (a.batch <= 1) return launch_gemv_b<FMT, CB, 1>(a, cfg, st);
    if (a.batch <= 2) return launch_gemv_b<FMT, CB, 2>(a, cfg, st);
    if (a.batch <= 4) return launch_gemv_b<FMT, CB, 4>(a, cfg, st);
    return launch_gemv_b<FMT, CB, 8>(a, cfg, st);
}

bool launch_gemv(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    const bool wide = (code_bytes_per_row(a.fmt, a.k) % 16) == 0;
    switch (a.fmt) {
        case kMXFP4: return launch_gemv_cb<kMXFP4, 16>(a, cfg, st);
        case kMXFP8: return launch_gemv_cb<kMXFP8, 16>(a, cfg, st);
        case kNVFP4: return wide ? launch_gemv_cb<kNVFP4, 16>(a, cfg, st) : launch_gemv_cb<kNVFP4, 8>(a, cfg, st);
    }
    return false;
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
