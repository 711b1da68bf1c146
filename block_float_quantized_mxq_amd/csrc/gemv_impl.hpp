// gemv_impl.hpp -- the dense GEMV kernel and its launcher for one format; each
// format is instantiated in its own translation unit (gemv_<format>.hip) so
// the instances compile in parallel.
#pragma once

#include <atomic>

#include "gemv_mfma.hpp"
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

// Passes each lane keeps in flight ahead of its arithmetic: one is enough with
// several waves per SIMD to switch between.
#ifndef MXQ_GEMV_AHEAD
#define MXQ_GEMV_AHEAD 1
#endif
constexpr int kGemvAhead = MXQ_GEMV_AHEAD;

// Largest LDS allocation for staged activations (x of the 25600-long rows
// of a down projection still fits three workgroups per CU).
constexpr int64_t kMaxXLds = 72 * 1024;

// Persistent grid of row tiles (rows_core.hpp): each tile is R rows per group
// of G lanes, split S ways along k (partials combined through LDS); the
// activations are read from LDS when they fit (staged once per workgroup)
// and otherwise from global memory, each chunk reused by the R rows.  Tiles
// tile, tile + gridDim.x, ... go to one workgroup as one stream of passes, so
// the GPU sweeps the matrix front to back; the first pass is in flight while
// the activations are staged.
template <int FMT, int CB, int B, int G, int S, int R, bool XL, bool MM>
__global__ __launch_bounds__(kThreads) void gemv_rows_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ gscale,
                                                             const uint16_t* __restrict__ x, float* __restrict__ y,
                                                             int64_t n, int64_t k, int batch, int64_t ntiles,
                                                             int contiguous) {
    using T = RowTile<G, S, R>;
    using E = RowEngine<FMT, CB, B, G, S, R, XL, false, MM>;
    __shared__ float red[E::RED_FLOATS];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
    const uint16_t* xs[B];
    float* ys[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        xs[b] = x + (int64_t)(b < batch ? b : 0) * k;
        ys[b] = b < batch ? y + (int64_t)b * n : nullptr;
    }
    const E eng(codes, scales, n, k);
    // tiles w, w + grid, w + 2 grid, ... (interleaved) or one contiguous range of
    // tiles per workgroup; the grid never exceeds the tile count
    const int64_t w = blockIdx.x, grid = gridDim.x;
    int64_t first, step, count;
    if (contiguous) {
        const int64_t per = ntiles / grid, rem = ntiles % grid;
        first = w * per + (w < rem ? w : rem);
        count = per + (w < rem ? 1 : 0);
        step = 1;
    } else {
        first = w;
        count = (ntiles - w + grid - 1) / grid;
        step = grid;
    }
    typename E::Cursor cur = eng.cursor(first * T::ROWS, step * T::ROWS, count, xs[0]);
    PassRing<typename E::Pass, kGemvAhead + 1> ring;
    eng.template prime<kGemvAhead>(cur, ring);
    const float gmul = (FMT == kNVFP4) ? gscale[0] : 1.0f;
    if constexpr (XL) stage_x<FMT, CB, B, MM>(xs, k, xlds);
    eng.template run<kGemvAhead>(cur, ring, xs, ys, gmul, red, xlds);
}

// Workgroups of `kernel` that fit on one CU with `lds` bytes of dynamic LDS
// (registers, waves and LDS together).  `cache` holds the last answer as
// (lds << 16) | count, per kernel instance.
template <typename K>
static int64_t resident_per_cu(K kernel, size_t lds, std::atomic<int64_t>& cache) {
    const int64_t c = cache.load(std::memory_order_relaxed);
    if (c >= 0 && (c >> 16) == (int64_t)lds) return c & 0xFFFF;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kThreads, lds) != hipSuccess) {
        (void)hipGetLastError();
        nb = 1;
    }
    if (nb < 1) nb = 1;
    cache.store(((int64_t)lds << 16) | nb, std::memory_order_relaxed);
    return nb;
}

template <int FMT, int CB, int B, int G, int S, int R, bool MM = false>
static void launch_rows_inst(const GemvArgs& a, int64_t per_cu, int grid_mode, hipStream_t st) {
    using T = RowTile<G, S, R>;
    static std::atomic<int64_t> occ_cache[2] = {{-1}, {-1}};
    const int64_t ntiles = (a.n + T::ROWS - 1) / T::ROWS;
    const bool xl = x_lds_bytes<FMT, CB>(a.k, B) <= kMaxXLds;
    const size_t lds = xl ? (size_t)x_lds_bytes<FMT, CB>(a.k, B) : 0;
    const auto kernel = xl ? gemv_rows_kernel<FMT, CB, B, G, S, R, true, MM>
                           : gemv_rows_kernel<FMT, CB, B, G, S, R, false, MM>;
    // Stay resident: no more workgroups per CU than fit at once.
    const int64_t fit = resident_per_cu(kernel, lds, occ_cache[xl ? 1 : 0]);
    if (per_cu > fit) per_cu = fit;
    // As many workgroups as are resident at once (measured: more bytes in
    // flight beats handing every workgroup the same number of tiles).
    const int64_t cap = (int64_t)a.cus * per_cu;
    int64_t blocks = ntiles < cap ? ntiles : cap;
    if (grid_mode == 1) {
        const int64_t rounds = (ntiles + cap - 1) / cap;
        blocks = (ntiles + rounds - 1) / rounds;
    } else if (grid_mode == 2) {
        blocks = ntiles;
    }
    const int contiguous = grid_mode == 3 ? 1 : 0;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), lds, st, a.codes, a.scales, a.gscale, a.x, a.y,
                       a.n, a.k, (int)a.batch, ntiles, contiguous);
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
            // 2 rows per lane, or 4 (each activation chunk reused 4 times) at
            // batch > 1 for very long rows or very many rows.
            g = 16;
            r = (B > 1 && (nchunks >= 512 || a.n >= 32768)) ? 4 : 2;
            sp = 1;
            int64_t best = -1;
            for (int cand : {1, 2, 4, 8}) {
                const int64_t per_lane10 = 10 * nchunks / (16 * cand);  // chunks per lane, x10
                const int64_t dist = per_lane10 > 50 ? per_lane10 - 50 : 50 - per_lane10;
                if (best < 0 || dist < best) { best = dist; sp = cand; }
            }
            if (r == 4 && sp == 8 && a.n < 2048) r = 2;
            if (r == 2 && sp == 8 && a.n < 1024) r = 1;
        }
    }
#define MXQ_ROWS_CASE(G_, S_, R_)                                         \
    if (g == G_ && sp == S_ && r == R_) {                                \
        launch_rows_inst<FMT, CB, B, G_, S_, R_>(a, occ, cfg.rows_grid, st); \
        return true;                                                     \
    }
    MXQ_ROWS_SHAPES(MXQ_ROWS_CASE)
#undef MXQ_ROWS_CASE
    return false;
}

// Matrix-mode settings (k split across waves s, four-row groups per lane r).
#define MXQ_MM_SHAPES(X) X(1, 4) X(2, 4) X(4, 4) X(2, 2) X(4, 2)

// Matrix mode (rows_core.hpp, MM) for batches 2 .. 4.  Settings measured on
// MI355X over the dense shapes (gate/up 51200 x 5120, down 5120 x 25600, QKV
// 7168 x 5120): k split across 2 waves, or 4 for rows of 512 chunks and more;
// 4 four-row groups per lane from batch 3 on long or many rows, else 2.  Batch
// 4: gate/up 41.6 -> 27.8 us, down 39.5 -> 23.1 us, QKV 10.9 -> 9.2 us against
// the FMA mode; batch 2: gate/up 27.6 -> 25.4 us, down 23.8 -> 18.7 us.  For
// down (800 chunks) the 4-way split beats the 2-way one at both batches
// (batch 2: 26.1 -> 19.7 us; batch 4: 27.2 -> 23.1 us with 4 groups per lane).
// A batch-4 down row set reads its activations from global memory (4 x 25600
// bf16 do not fit the LDS); carrying them with the passes, loaded as far ahead
// as the weights, measured slower (23.1 -> 24.8 us), so they are read on use.
template <int FMT, int CB, int B>
static bool launch_rows_mm(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    int sp = cfg.mm_s, r = cfg.mm_r;
    const int64_t occ = cfg.rows_occ > 0 ? cfg.rows_occ : 8;
    if (sp == 0 || r == 0) {
        const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
        sp = nchunks >= 512 ? 4 : 2;
        r = (a.batch >= 3 && (a.n >= 16384 || nchunks >= 512)) ? 4 : 2;
    }
#define MXQ_MM_CASE(S_, R_)                                                    \
    if (sp == S_ && r == R_) {                                                \
        launch_rows_inst<FMT, CB, B, 16, S_, R_, true>(a, occ, cfg.rows_grid, st); \
        return true;                                                          \
    }
    MXQ_MM_SHAPES(MXQ_MM_CASE)
#undef MXQ_MM_CASE
    return false;
}

template <int FMT, int CB>
static bool launch_gemv_cb(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    // Batch 1: the FMA mode (HBM bound, fastest on every dense shape).  Batch
    // 2 .. 4: matrix mode, where the FMA mode's dot2 per two weights per
    // vector makes the vector ALU the bound.  From batch 5: the matrix-unit
    // GEMV (16 vectors per MFMA column set).
    if (cfg.path == 4 || (cfg.path == 0 && a.batch >= 2 && a.batch <= 4)) {
        if (a.batch <= 1) return launch_rows_mm<FMT, CB, 1>(a, cfg, st);
        if (a.batch <= 2) return launch_rows_mm<FMT, CB, 2>(a, cfg, st);
        if (a.batch <= 4) return launch_rows_mm<FMT, CB, 4>(a, cfg, st);
    }
    const bool mfma = cfg.path == 1 || (cfg.path == 0 && a.batch >= 5);
    if (mfma && a.k % 32 == 0) return launch_gemv_mfma<FMT>(a, cfg, st);
    if (a.batch <= 1) return launch_rows_b<FMT, CB, 1>(a, cfg, st);
    if (a.batch <= 2) return launch_rows_b<FMT, CB, 2>(a, cfg, st);
    if (a.batch <= 4) return launch_rows_b<FMT, CB, 4>(a, cfg, st);
    return launch_rows_b<FMT, CB, 8>(a, cfg, st);
}

}  // namespace mxq
