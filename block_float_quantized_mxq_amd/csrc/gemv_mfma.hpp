// gemv_mfma.hpp -- dense GEMV on the matrix unit, for small batches.
//
// y[b][r] = sum_k W[r][k] * x[b][k] for batch <= 16 (fp32, or bf16 rounded to
// nearest even for the small-m prefill GEMM), written as a 16 x 16 x 32
// bf16 MFMA per k step: the A operand is 16 weight rows decoded from their
// codes (block_operand.hpp), the B operand is x with one column per batch
// entry (columns past the batch hold zeros), and the fp32 accumulator holds
// y for 16 rows x 16 columns.  With the FMA path (rows_core.hpp) every batch
// entry costs one dot2 per two weights, so at batch 4 the vector ALU rather
// than HBM sets the pace; here the contraction runs on the matrix unit and the
// vector ALU only decodes (half an instruction per weight, whatever the batch).
//
// Lane l of a wave serves row l % 16 and k group g = l / 16.  In a pass each
// lane loads whole 32-element blocks of its row: blocks p0 + g + 4u
// (u < U), so one load instruction covers 64 contiguous code bytes of each of
// the wave's 16 rows (MXFP4 / NVFP4, U = 2: two instructions make a 128-byte
// line) or 128 bytes (E4M3, U = 1, two 16-byte loads per block).  The B
// operand lane with the same g reads the matching 16 bytes of x, so both
// operands take the same k permutation and the MFMA sums the right products.
//
// Work split: a workgroup of NW waves owns tiles of NW / KS row blocks of 16
// rows (R blocks per wave, sharing the B operands); the KS waves of one row
// block split k and add their partial sums through LDS in a fixed order (no
// atomics: the result is the same on every run).  Tiles tile, tile + grid,
// ... go to one workgroup, and each wave streams its passes across tile
// boundaries one pass ahead: the loads of pass p + 1 (codes, scales and x,
// which the caches serve) are issued before the MFMAs of pass p.  Lanes past
// the end of a k range load a valid block again and zero their operands.
#pragma once

#include "block_operand.hpp"
#include "kernels.hpp"

namespace mxq {

typedef float f32x4m_t __attribute__((ext_vector_type(4)));

template <int FMT>
struct MfmaShape {
    static constexpr int U = (FMT == kMXFP8) ? 1 : 2;  // blocks per lane per row per pass
    static constexpr int BPP = 4 * U;                   // blocks per row per pass
    static constexpr int CBB = (FMT == kMXFP8) ? 32 : 16;  // code bytes per block
};

// One pass of one lane: U blocks of each of its R rows, and the x pieces of
// those blocks (4 k steps of 8 bf16 each).
template <int FMT, int R>
struct MPass {
    WFrag<FMT> w[R][MfmaShape<FMT>::U];
    u32x4g_t x[MfmaShape<FMT>::U][4];
    uint32_t valid;  // bit u: block u lies inside the wave's k range
};

// Loads block `blk` of one row (blk must be a valid block of the row): codes
// with the nontemporal hint (read once), scale bytes through the caches.
template <int FMT>
__device__ __forceinline__ void load_block(const uint8_t* crow, const uint8_t* srow, int64_t blk, WFrag<FMT>& f) {
    const u32x4g_t* q = reinterpret_cast<const u32x4g_t*>(crow + blk * MfmaShape<FMT>::CBB);
    const u32x4g_t v0 = __builtin_nontemporal_load(q);
    f.w[0] = v0[0]; f.w[1] = v0[1]; f.w[2] = v0[2]; f.w[3] = v0[3];
    if constexpr (FMT == kMXFP8) {
        const u32x4g_t v1 = __builtin_nontemporal_load(q + 1);
        f.w[4] = v1[0]; f.w[5] = v1[1]; f.w[6] = v1[2]; f.w[7] = v1[3];
    }
    if constexpr (FMT == kNVFP4) f.s = (uint32_t)srow[2 * blk] | ((uint32_t)srow[2 * blk + 1] << 8);
    else f.s = srow[blk];
}

template <int FMT, int R, int KS, int NW>
struct MfmaTile {
    static constexpr int WR = NW / KS;             // row blocks (of 16 x R rows) per tile
    static constexpr int ROWS = WR * R * 16;       // rows per tile
    static constexpr int THREADS = NW * 64;
    // LDS for the k-split sums: 2 buffers x NW waves x R blocks x 64 lanes x 4 floats
    static constexpr int RED_FLOATS = KS > 1 ? 2 * NW * R * 256 : 1;
};

// x rows staged in LDS are padded by 8 bf16 so that the B operand reads of
// different batch columns start in different banks.
__host__ __device__ constexpr int64_t mfma_x_stride(int64_t k) { return k + 8; }

template <int FMT, int R, int KS, int NW, bool XL>
__global__ __launch_bounds__(NW * 64) void gemv_mfma_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gscale,
                                                            const uint16_t* __restrict__ x, float* __restrict__ y,
                                                            int64_t n, int64_t k, int batch, int64_t ntiles,
                                                            int y_bf16) {
    using Sh = MfmaShape<FMT>;
    using Ti = MfmaTile<FMT, R, KS, NW>;
    using P = MPass<FMT, R>;
    __shared__ __attribute__((aligned(16))) float red[Ti::RED_FLOATS];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];

    const int wave = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int lr = l & 15;   // row within a block of 16; also the batch column of the B operand
    const int g = l >> 4;    // k group
    const int wr = wave / KS, kp = wave % KS;

    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t sbytes = k / block_elems(FMT);
    const int64_t nblk = k / 32;
    // k range of this wave: blocks [kb0, kb1), whole passes except at the row end
    const int64_t part = ((nblk + KS - 1) / KS + Sh::BPP - 1) / Sh::BPP * Sh::BPP;
    const int64_t kb0 = (int64_t)kp * part;
    const int64_t kb1 = kb0 + part < nblk ? kb0 + part : nblk;
    const int64_t len = kb1 > kb0 ? kb1 - kb0 : 0;
    const int64_t ppt = len > 0 ? (len + Sh::BPP - 1) / Sh::BPP : 1;  // passes per tile (at least one)
    const int64_t last_blk = kb1 > kb0 ? kb1 - 1 : 0;                 // a valid block to read when out of range

    const int64_t tile0 = blockIdx.x;
    const int64_t count = (ntiles - tile0 + gridDim.x - 1) / gridDim.x;
    const int64_t total = count * ppt;
    const int xcol = lr < batch ? lr : 0;  // B operand column (lanes past the batch read x[0], then zero)
    const bool xlive = lr < batch;
    const uint16_t* xrow = x + (int64_t)xcol * k;

    // load cursor
    int64_t tl = 0, il = 0;
    const uint8_t* crow[R];
    const uint8_t* srow[R];
    auto set_rows = [&](int64_t t) {
        const int64_t row0 = (tile0 + t * gridDim.x) * Ti::ROWS + (int64_t)wr * R * 16;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t row = row0 + r * 16 + lr;
            row = row < n ? row : n - 1;
            crow[r] = codes + row * rowbytes;
            srow[r] = scales + row * sbytes;
        }
    };
    set_rows(0);

    auto load = [&](P& p) {
        const int64_t pb = kb0 + il * Sh::BPP + g;
        uint32_t valid = 0;
#pragma unroll
        for (int u = 0; u < Sh::U; ++u) {
            const int64_t b = pb + 4 * u;
            const bool ok = b < kb1 && tl < count;
            valid |= (ok ? 1u : 0u) << u;
            const int64_t bb = ok ? b : last_blk;
#pragma unroll
            for (int r = 0; r < R; ++r) load_block<FMT>(crow[r], srow[r], bb, p.w[r][u]);
            if constexpr (!XL) {
                const u32x4g_t* xp = reinterpret_cast<const u32x4g_t*>(xrow + bb * 32);
#pragma unroll
                for (int s = 0; s < 4; ++s) p.x[u][s] = xp[s];
            } else {
                p.x[u][0][0] = (uint32_t)bb;  // block index for the LDS read
            }
        }
        p.valid = valid;
        if (++il == ppt) {
            il = 0;
            ++tl;
            set_rows(tl < count ? tl : 0);
        }
    };

    // compute cursor
    int64_t tc = 0, ic = 0;
    f32x4m_t acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = f32x4m_t{0.f, 0.f, 0.f, 0.f};
    const float gmul = (FMT == kNVFP4) ? gscale[0] : 1.0f;

    auto store = [&](int64_t idx, float v) {
        if (y_bf16) reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
        else y[idx] = v;
    };
    auto finish = [&]() {
        const int64_t rowt = (tile0 + tc * gridDim.x) * Ti::ROWS + (int64_t)wr * R * 16;
        if constexpr (KS == 1) {
            if (xlive) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t row = rowt + r * 16 + 4 * g + i;
                        if (row < n) store((int64_t)lr * n + row, acc[r][i] * gmul);
                    }
            }
        } else {
            float* rb = red + (tc & 1) * (NW * R * 256);
#pragma unroll
            for (int r = 0; r < R; ++r)
                *reinterpret_cast<f32x4m_t*>(rb + ((wave * R + r) * 64 + l) * 4) = acc[r];
            lds_barrier();
            if (kp == 0 && xlive) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    f32x4m_t v = acc[r];
#pragma unroll
                    for (int q = 1; q < KS; ++q) v += *reinterpret_cast<const f32x4m_t*>(rb + (((wave + q) * R + r) * 64 + l) * 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t row = rowt + r * 16 + 4 * g + i;
                        if (row < n) store((int64_t)lr * n + row, v[i] * gmul);
                    }
                }
            }
            // the other buffer is rewritten only after the next tile's barrier
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = f32x4m_t{0.f, 0.f, 0.f, 0.f};
    };

    auto compute = [&](const P& p) {
        // MXFP8 passes holding a block with an E8M0 byte below kMx8Lift run the
        // split form (block_operand.hpp); the branch is uniform over the wave
        bool lifted = false;
        if constexpr (FMT == kMXFP8) {
            bool lo = false;
#pragma unroll
            for (int u = 0; u < Sh::U; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r) lo = lo || (((p.valid >> u) & 1u) && frag_lifted<FMT>(p.w[r][u]));
            lifted = __ballot(lo) != 0;
        }
#pragma unroll
        for (int u = 0; u < Sh::U; ++u) {
            const bool ok = (p.valid >> u) & 1u;
            const bool xo = ok && xlive;
            bf16x8_t b[4];
            if constexpr (XL) {
                // only the lanes of live batch columns read LDS
                u32x4g_t v[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
                if (xo) {
                    const u32x4g_t* xp = reinterpret_cast<const u32x4g_t*>(xlds) +
                                         ((int64_t)lr * mfma_x_stride(k) + (int64_t)p.x[u][0][0] * 32) / 8;
#pragma unroll
                    for (int s = 0; s < 4; ++s) v[s] = xp[s];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) b[s] = __builtin_bit_cast(bf16x8_t, v[s]);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const u32x4g_t v = p.x[u][s];
                    b[s] = __builtin_bit_cast(bf16x8_t, u32x4g_t{xo ? v[0] : 0u, xo ? v[1] : 0u, xo ? v[2] : 0u, xo ? v[3] : 0u});
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // a block outside the k range decodes as zeros with a unit scale
                WFrag<FMT> f = p.w[r][u];
#pragma unroll
                for (int d = 0; d < WFrag<FMT>::DW; ++d) f.w[d] = ok ? f.w[d] : 0u;
                f.s = ok ? f.s : (FMT == kNVFP4 ? 0x3838u : 127u);
                if constexpr (FMT == kMXFP8) {
                    if (lifted) {
                        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 0, false>(f), b[0], acc[r], 0, 0, 0);
                        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 1, false>(f), b[1], acc[r], 0, 0, 0);
                        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 2, false>(f), b[2], acc[r], 0, 0, 0);
                        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 3, false>(f), b[3], acc[r], 0, 0, 0);
                        f32x4m_t t = {0.f, 0.f, 0.f, 0.f};
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 0, true>(f), b[0], t, 0, 0, 0);
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 1, true>(f), b[1], t, 0, 0, 0);
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 2, true>(f), b[2], t, 0, 0, 0);
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 3, true>(f), b[3], t, 0, 0, 0);
                        acc[r] += t * kMx8Unlift;
                        continue;
                    }
                }
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 0>(f), b[0], acc[r], 0, 0, 0);
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 1>(f), b[1], acc[r], 0, 0, 0);
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 2>(f), b[2], acc[r], 0, 0, 0);
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 3>(f), b[3], acc[r], 0, 0, 0);
            }
        }
        if (++ic == ppt) {
            finish();
            ic = 0;
            ++tc;
        }
    };

    P pa, pb;
    load(pa);
    if constexpr (XL) {
        // stage x[batch][k] (16-byte pieces) while the first pass is in flight
        const int64_t pieces = k / 8;
        for (int b = 0; b < batch; ++b) {
            const u32x4g_t* src = reinterpret_cast<const u32x4g_t*>(x + (int64_t)b * k);
            u32x4g_t* dst = reinterpret_cast<u32x4g_t*>(xlds) + b * mfma_x_stride(k) / 8;
            for (int64_t t = threadIdx.x; t < pieces; t += NW * 64) dst[t] = src[t];
        }
        lds_barrier();
    }
    int64_t q = 0;
    for (; q + 2 <= total; q += 2) {
        load(pb);
        compute(pa);
        load(pa);
        compute(pb);
    }
    if (q < total) compute(pa);
}

// Largest LDS allocation for staged x (beyond it x is read through the caches).
constexpr int64_t kMfmaMaxXLds = 64 * 1024;

template <int FMT, int R, int KS, int NW>
static void launch_mfma_inst(const GemvArgs& a, int64_t per_cu, hipStream_t st) {
    using Ti = MfmaTile<FMT, R, KS, NW>;
    const int64_t ntiles = (a.n + Ti::ROWS - 1) / Ti::ROWS;
    const int64_t cap = (int64_t)a.cus * per_cu;
    const int64_t blocks = ntiles < cap ? ntiles : cap;
    const int64_t lds = a.batch * mfma_x_stride(a.k) * 2;
    if (lds <= kMfmaMaxXLds)
        hipLaunchKernelGGL((gemv_mfma_kernel<FMT, R, KS, NW, true>), dim3((unsigned)blocks), dim3(Ti::THREADS),
                           (size_t)lds, st, a.codes, a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch, ntiles,
                           a.y_bf16);
    else
        hipLaunchKernelGGL((gemv_mfma_kernel<FMT, R, KS, NW, false>), dim3((unsigned)blocks), dim3(Ti::THREADS), 0,
                           st, a.codes, a.scales, a.gscale, a.x, a.y, a.n, a.k, (int)a.batch, ntiles, a.y_bf16);
}

// Compiled (rows per wave R, k split KS, waves per workgroup NW) settings.
#define MXQ_MFMA_SHAPES(X) X(1, 1, 4) X(2, 1, 4) X(4, 1, 4) X(1, 2, 4) X(1, 4, 4) X(2, 4, 4) X(4, 4, 4) X(2, 8, 8)

// MFMA GEMV for MX formats (and NVFP4 with k a multiple of 32).  Settings come
// from the shape unless cfg.mfma_ks > 0 (tuning override).
template <int FMT>
static bool launch_gemv_mfma(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    int r = cfg.mfma_r, ks = cfg.mfma_ks, nw = cfg.mfma_nw;
    int64_t occ = cfg.mfma_occ;
    if (ks <= 0) {
        // measured on MI355X: two row blocks per wave, k split four ways
        r = 2;
        ks = 4;
        nw = 4;
        occ = 2;
    }
    if (occ <= 0) occ = nw >= 8 ? 1 : 2;
#define MXQ_MFMA_CASE(R_, KS_, NW_)                                 \
    if (r == R_ && ks == KS_ && nw == NW_) {                       \
        launch_mfma_inst<FMT, R_, KS_, NW_>(a, occ, st);           \
        return true;                                               \
    }
    MXQ_MFMA_SHAPES(MXQ_MFMA_CASE)
#undef MXQ_MFMA_CASE
    return false;
}

}  // namespace mxq
