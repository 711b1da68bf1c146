// gemv_impl.hpp -- the dense GEMV kernel and its launcher for one format; each
// format is instantiated in its own translation unit (gemv_<format>.hip) so
// the instances compile in parallel.
#pragma once

#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

// Largest LDS allocation for staged activations (keeps two workgroups per CU
// within the 160 KB of LDS).
constexpr int64_t kMaxXLds = 72 * 1024;

// Persistent grid of row tiles (rows_core.hpp): each tile is R rows per group
// of G lanes, split S ways along k (partials combined through LDS); the
// activations are read from LDS when they fit (staged once per workgroup)
// and otherwise from global memory, each chunk reused by the R rows.  Tile
// tile, tile + gridDim.x, ... go to one workgroup, so the GPU sweeps the
// matrix front to back.
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
static void launch_rows_inst(const GemvArgs& a, int64_t per_cu, hipStream_t st) {
    using T = RowTile<G, S, R>;
    const int64_t ntiles = (a.n + T::ROWS - 1) / T::ROWS;
    const bool xl = x_lds_bytes<FMT, CB>(a.k, B) <= kMaxXLds;
    const size_t lds = xl ? (size_t)x_lds_bytes<FMT, CB>(a.k, B) : 0;
    // stay resident: no more workgroups than fit in 160 KB of LDS per CU
    const int64_t fit = (160 * 1024) / ((int64_t)lds + 4096);
    if (per_cu > fit) per_cu = fit > 0 ? fit : 1;
    const int64_t cap = 256 * per_cu;
    const int64_t blocks = ntiles < cap ? ntiles : cap;
    if (xl)
        hipLaunchKernelGGL((gemv_rows_kernel<FMT, CB, B, G, S, R, true>), dim3((unsigned)blocks), dim3(kThreads), lds,
                           st, a.codes, a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch, ntiles);
    else
        hipLaunchKernelGGL((gemv_rows_kernel<FMT, CB, B, G, S, R, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           st, a.codes, a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch, ntiles);
}

// Row-tile settings (lanes per row g, k split s, rows per lane r, workgroups
// per CU) for a shape; rows_cfg.g == 0 selects them from the shape.
template <int FMT, int CB, int B>
static bool launch_rows_b(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
    int g = cfg.rows_g, sp = cfg.rows_s, r = cfg.rows_r;
    const int64_t occ = cfg.rows_occ > 0 ? cfg.rows_occ : 8;
    if (g == 0) {
        if (nchunks < 8) { g = 4; sp = 1; r = 1; }
        else if (nchunks < 16) { g = 8; sp = 1; r = 1; }
        else {
            // Measured on MI355X: about 5 chunks per lane per row pass is best;
            // 4 rows per lane (each activation chunk reused 4 times) wins at
            // batch > 1 and for very long rows.
            g = 16;
            r = (B > 1 || nchunks >= 512) ? 4 : 1;
            sp = 1;
            int64_t best = -1;
            for (int cand : {1, 2, 4, 8}) {
                const int64_t per_lane10 = 10 * nchunks / (16 * cand);  // chunks per lane, x10
                const int64_t dist = per_lane10 > 50 ? per_lane10 - 50 : 50 - per_lane10;
                if (best < 0 || dist < best) { best = dist; sp = cand; }
            }
            if (r == 4 && sp == 8 && a.n < 2048) r = 2;
        }
    }
#define MXQ_ROWS_CASE(G_, S_, R_)                                         \
    if (g == G_ && sp == S_ && r == R_) {                                \
        launch_rows_inst<FMT, CB, B, G_, S_, R_>(a, occ, st);            \
        return true;                                                     \
    }
    MXQ_ROWS_SHAPES(MXQ_ROWS_CASE)
#undef MXQ_ROWS_CASE
    return false;
}

template <int FMT, int CB>
static bool launch_gemv_cb(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    if (a.batch <= 1) return launch_rows_b<FMT, CB, 1>(a, cfg, st);
    if (a.batch <= 2) return launch_rows_b<FMT, CB, 2>(a, cfg, st);
    if (a.batch <= 4) return launch_rows_b<FMT, CB, 4>(a, cfg, st);
    return launch_rows_b<FMT, CB, 8>(a, cfg, st);
}

}  // namespace mxq
