// gemv_impl.hpp -- launcher of the dense GEMV stream kernel (gemv_stream.hpp)
// for one format; each format is instantiated in its own translation unit
// (gemv_<format>.hip) so the instances compile in parallel.
#pragma once

#include "gemv_stream.hpp"
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

// Largest LDS allocation for staged activations (keeps two workgroups per CU
// within the 160 KB of LDS).
constexpr int64_t kMaxXLds = 72 * 1024;

template <int FMT, int CB, int B, int G, int P, int D, bool XL>
static void launch_stream_inst(const GemvArgs& a, int64_t wgs, hipStream_t st) {
    const int64_t per_wg = kThreads / G;
    const int64_t nblocks = (a.n + P - 1) / P;
    const int64_t need = (nblocks + per_wg - 1) / per_wg;  // one block per group at most
    const int64_t blocks = wgs < need ? wgs : need;
    const size_t lds = XL ? (size_t)x_lds_bytes<FMT, CB>(a.k, B) : 0;
    hipLaunchKernelGGL((gemv_stream_kernel<FMT, CB, B, G, P, D, XL>), dim3((unsigned)blocks), dim3(kThreads), lds, st,
                       a.codes, a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch);
}

// Rows per block for G lanes: the smallest P with P * nchunks a multiple of
// G (0 if none of the compiled P values fits, or the row has fewer than G chunks).
inline int stream_rows_per_block(int64_t nchunks, int g) {
    if (nchunks < g) return 0;
    for (int p : {1, 2, 4}) if ((p * nchunks) % g == 0) return p;
    return 0;
}

template <int FMT, int CB, int B>
static bool launch_gemv_b(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    if (!cfg.xl || x_lds_bytes<FMT, CB>(a.k, B) > kMaxXLds) return false;
    const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
    const int p = stream_rows_per_block(nchunks, cfg.g);
    const int64_t wgs = cfg.wgs > 0 ? cfg.wgs : 1024;
#define MXQ_STREAM_CASE(G_, D_)                                                           \
    if (cfg.g == G_ && cfg.d == D_) {                                                    \
        if (p == 1) launch_stream_inst<FMT, CB, B, G_, 1, D_, true>(a, wgs, st);         \
        else if (p == 2) launch_stream_inst<FMT, CB, B, G_, 2, D_, true>(a, wgs, st);    \
        else if (p == 4) launch_stream_inst<FMT, CB, B, G_, 4, D_, true>(a, wgs, st);    \
        else return false;                                                               \
        return true;                                                                     \
    }
    MXQ_STREAM_SHAPES(MXQ_STREAM_CASE)
#undef MXQ_STREAM_CASE
    return false;
}

// ---- fallback: row tiles through rows_core (any k, any batch) -------------
//
// Used when the stream kernel does not apply: activations too large for LDS
// (long rows at batch > 1) or rows whose chunk count fits no block shape.
// Persistent grid of row tiles; each tile is R rows per group of G lanes,
// split S ways along k (partials combined through LDS), activations read from
// LDS when they fit and otherwise from global memory, reused by the R rows.
template <int FMT, int CB, int B, int G, int S, int R, bool XL>
__global__ __launch_bounds__(kThreads) void gemv_rows_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ gscale,
                                                             const uint16_t* __restrict__ x, float* __restrict__ y,
                                                             int64_t n, int64_t k, int batch, int64_t ntiles) {
    using T = RowTile<G, S, R>;
    __shared__ float red[S > 1 ? S * T::ROWSETS * R * B : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
    const uint16_t* xs[B];
    float* ys[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        xs[b] = x + (int64_t)(b < batch ? b : 0) * k;
        ys[b] = b < batch ? y + (int64_t)b * n : nullptr;
    }
    const float gmul = (FMT == kNVFP4) ? gscale[0] : 1.0f;
    if constexpr (XL) stage_x<FMT, CB, B>(xs, k, xlds);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x)
        rows_core<FMT, CB, B, G, S, R, XL>(codes, scales, n, k, tile * T::ROWS, xs, ys, gmul, red, xlds);
}

template <int FMT, int CB, int B, int G, int S, int R>
static void launch_rows_inst(const GemvArgs& a, hipStream_t st) {
    using T = RowTile<G, S, R>;
    const int64_t ntiles = (a.n + T::ROWS - 1) / T::ROWS;
    const bool xl = x_lds_bytes<FMT, CB>(a.k, B) <= kMaxXLds;
    const size_t lds = xl ? (size_t)x_lds_bytes<FMT, CB>(a.k, B) : 0;
    const int64_t cap = xl && lds > 40 * 1024 ? 512 : 1024;  // stay resident: LDS is 160 KB per CU
    const int64_t blocks = ntiles < cap ? ntiles : cap;
    if (xl)
        hipLaunchKernelGGL((gemv_rows_kernel<FMT, CB, B, G, S, R, true>), dim3((unsigned)blocks), dim3(kThreads), lds,
                           st, a.codes, a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch, ntiles);
    else
        hipLaunchKernelGGL((gemv_rows_kernel<FMT, CB, B, G, S, R, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           st, a.codes, a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch, ntiles);
}

template <int FMT, int CB, int B>
static bool launch_rows_b(const GemvArgs& a, hipStream_t st) {
    const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
    if (nchunks < 8) { launch_rows_inst<FMT, CB, B, 4, 1, 1>(a, st); return true; }
    if (nchunks < 16) { launch_rows_inst<FMT, CB, B, 8, 1, 1>(a, st); return true; }
    // rows per lane: reuse each activation chunk across 4 rows at batch > 1;
    // split k until the grid has about 1024 tiles, keeping >= 2 chunks per lane
    if (B == 1) {
        if (a.n / 16 >= 1024 || nchunks < 64) launch_rows_inst<FMT, CB, B, 16, 1, 1>(a, st);
        else if (a.n / 8 >= 1024 || nchunks < 128) launch_rows_inst<FMT, CB, B, 16, 2, 1>(a, st);
        else if (a.n / 4 >= 1024 || nchunks < 256) launch_rows_inst<FMT, CB, B, 16, 4, 1>(a, st);
        else launch_rows_inst<FMT, CB, B, 16, 8, 1>(a, st);
    } else {
        if (a.n / 64 >= 1024 || nchunks < 64) launch_rows_inst<FMT, CB, B, 16, 1, 4>(a, st);
        else if (a.n / 32 >= 1024 || nchunks < 128) launch_rows_inst<FMT, CB, B, 16, 2, 4>(a, st);
        else launch_rows_inst<FMT, CB, B, 16, 8, 4>(a, st);
    }
    return true;
}

template <int FMT, int CB, int B>
static bool launch_any_b(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    if (launch_gemv_b<FMT, CB, B>(a, cfg, st)) return true;
    return launch_rows_b<FMT, CB, B>(a, st);
}

template <int FMT, int CB>
static bool launch_gemv_cb(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    if (a.batch <= 1) return launch_any_b<FMT, CB, 1>(a, cfg, st);
    if (a.batch <= 2) return launch_any_b<FMT, CB, 2>(a, cfg, st);
    if (a.batch <= 4) return launch_any_b<FMT, CB, 4>(a, cfg, st);
    return launch_any_b<FMT, CB, 8>(a, cfg, st);
}

}  // namespace mxq
