// gemm.hip -- prefill GEMM on block-float weights: Y[m][i] = sum_k X[m][k] * W[i][k].
//
// Prefill is compute bound ("The memory wall" section of the "MLxcel 0.8
// release" post, slide 15 of the talk); the pages' fast path decodes the
// quantized weights on the GPU and feeds the matrix unit ("Decoding block-float
// formats in software", slide 12).  Here:
//
//  * A workgroup (8 waves, 2 x 4) owns a 256 x 256 tile of Y; each wave owns
//    128 x 64 = 4 x 2 bf16 MFMA 32x32x16 tiles with fp32 accumulators (128
//    accumulator registers), so two waves share each SIMD and one issues
//    MFMAs while the other waits on memory, decodes or stores.
//  * Only X goes through LDS: per 64-wide k slice the workgroup stages the
//    256 x 64 bf16 block of X (double buffered, rows padded by 16 bytes so the
//    operand reads of 16 rows hit distinct banks).
//  * W never goes through LDS: each wave loads the codes of its own 128
//    columns from global memory (L2 resident: the workgroups of one XCD share
//    them) and decodes them straight into MFMA B operands with the gfx950
//    scaled conversion.  Within a slice the k order is permuted identically
//    for A and B (the sum does not depend on it): in k step s the lanes of
//    half g take k = g*32 + s*8 .. +7, so each lane's codes for the whole
//    slice are one 32-element block, one 16-byte load (32 for E4M3) with one
//    scale byte.  E8M0 scales go into the conversion (exact at every byte;
//    MXFP8 fragments with a byte below kMx8Lift are split, block_operand.hpp);
//    NVFP4's E4M3 scales multiply in fp32 (q * s has at most 6 significant
//    bits, so its bf16 is exact).
//  * Slices are pipelined: while slice s is multiplied, slice s+1's X waits in
//    registers (stored to the other LDS buffer after the MFMAs) and its W
//    codes are already in registers; slice s+2 is requested after them.  One
//    barrier per slice, waiting for LDS traffic only (the requests for slice
//    s+2 stay in flight across it).
//  * Tiles are ordered so that the 32 workgroups resident on one XCD (the
//    dispatcher deals workgroup i to XCD i mod 8) work on a compact block of
//    4 x 8 tiles and share their X and W slices in that XCD's L2.
//  * A last, partly filled round of tiles runs as 128 x 128 tiles (the same
//    kernel with 2 x 1 MFMA blocks per wave) in a second launch (below).
//  * The NVFP4 per-tensor scale multiplies the fp32 result; the bf16 output is
//    rounded to nearest even from that fp32 value.
#include <atomic>
#include <type_traits>

#include "kernels.hpp"
#include "mxq_device.hpp"
#include "block_operand.hpp"
#include "rows_core.hpp"

namespace mxq {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kGemmThreads = 512;

// Slice shape per format: 64 k (each lane's W share one 32-element block,
// 16 bytes of E2M1 codes), or 32 k for E4M3 (a 16-element half block, 16
// bytes: a 32-byte share leaves too few registers for the pipelined slices).
template <int FMT, int BM = kBM>
struct GemmSlice {
    static constexpr int BK = FMT == kMXFP8 ? 32 : 64;
    static constexpr int KE = BK / 2;                         // k per lane per fragment
    static constexpr int STEPS = BK / 16;                     // MFMA k steps per slice
    static constexpr int XSTRIDE = BK + 8;                    // bf16 per LDS row of X (16-byte pad)
    static constexpr int XTILE = BM * XSTRIDE;                // per buffer
    static constexpr int PPR = BK / 8;                        // 16-byte pieces per row
    static constexpr int XPIECES = BM * BK / 8 / kGemmThreads;
    static_assert(XPIECES >= 1 && BM * BK / 8 % kGemmThreads == 0, "whole X pieces per thread");
};

// Tile coordinates of workgroup b (XCD-aware grouped order): consecutive
// "local" indices of one XCD walk a GM-tall column strip of tiles, n fastest.
__device__ __forceinline__ void tile_of(int64_t b, int64_t mt, int64_t nt, int64_t& tm, int64_t& tn) {
    const int64_t total = mt * nt;
    const int64_t per_xcd = (total + 7) / 8;
    const int64_t xcd = b % 8, local = b / 8;
    int64_t t = xcd * per_xcd + local;  // tiles [xcd*per_xcd, ...) belong to one XCD
    if (t >= total) t = b;              // uneven tail: plain order (each tile once: see launcher)
    constexpr int64_t GM = 4;
    const int64_t group = t / (GM * nt);
    const int64_t first_m = group * GM;
    const int64_t gm = (mt - first_m) < GM ? (mt - first_m) : GM;
    const int64_t in = t % (GM * nt);
    tm = first_m + in % gm;
    tn = in / gm;
}

// TI x TJ: the 32x32 MFMA blocks of each wave (4 x 2: 256 x 256 tiles; 2 x 1:
// 128 x 128 tiles).  The launch covers output columns noff .. noff + ncols - 1.
template <int FMT, bool ROW8, int TI = 4, int TJ = 2>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gscale,
                                                            const uint16_t* __restrict__ x, void* __restrict__ yv,
                                                            int y_bf16, int64_t m, int64_t n, int64_t k,
                                                            int xcd_order, int64_t noff, int64_t ncols) {
    constexpr int BM = 2 * 32 * TI, BN = 4 * 32 * TJ;
    using GS = GemmSlice<FMT, BM>;
    constexpr int kBK = GS::BK, kXStride = GS::XSTRIDE, kXTileElems = GS::XTILE, kXPieces = GS::XPIECES;
    constexpr int kPPR = GS::PPR;
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_lds[];  // [2][kBM][kXStride]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;  // rows wm*32*TI .. +32*TI-1, columns wn*32*TJ .. +32*TJ-1
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t mt = (m + BM - 1) / BM, nt = (ncols + BN - 1) / BN;
    int64_t tm, tn;
    if (xcd_order) tile_of(blockIdx.x, mt, nt, tm, tn);
    else { tm = blockIdx.x / nt; tn = blockIdx.x % nt; }
    const int64_t m0 = tm * BM, n0 = noff + tn * BN;
    const int64_t nend = noff + ncols;  // columns of this launch end here (rows of W past it are not read)

    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t sbytes = k / block_elems(FMT);

    // X loader: piece p = tid + kGemmThreads*u is row p/kPPR, 16-byte column p%kPPR of the slice.
    const uint16_t* xrow[kXPieces];
#pragma unroll
    for (int u = 0; u < kXPieces; ++u) {
        const int p = tid + kGemmThreads * u;
        int64_t r = m0 + p / kPPR;
        r = r < m ? r : m - 1;  // rows past m read row m-1; their outputs are not written
        xrow[u] = x + r * k + (p % kPPR) * 8;
    }
    // W rows of this lane's TJ fragments (columns wn*32*TJ + j*32 + l32).
    const uint8_t* crow[TJ];
    const uint8_t* srow[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        int64_t r = n0 + wn * 32 * TJ + j * 32 + l32;
        r = r < nend ? r : nend - 1;
        crow[j] = codes + r * rowbytes;
        srow[j] = scales + r * sbytes;
    }

    u32x4g_t xr[kXPieces];
    auto load_x = [&](int64_t k0) {
#pragma unroll
        for (int u = 0; u < kXPieces; ++u) {
            const int p = tid + kGemmThreads * u;
            if (k0 + (p % kPPR) * 8 < k) xr[u] = *reinterpret_cast<const u32x4g_t*>(xrow[u] + k0);
            else xr[u] = u32x4g_t{0u, 0u, 0u, 0u};
        }
    };
    auto store_x = [&](int buf) {
        uint16_t* dst = xs_lds + buf * kXTileElems;
#pragma unroll
        for (int u = 0; u < kXPieces; ++u) {
            const int p = tid + kGemmThreads * u;
            *reinterpret_cast<u32x4g_t*>(dst + (p / kPPR) * kXStride + (p % kPPR) * 8) = xr[u];
        }
    };
    using Frag = WFrag<FMT, GS::KE>;
    auto load_w = [&](int64_t k0, Frag (&wf)[TJ]) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) load_wfrag<FMT, GS::KE, ROW8>(crow[j], srow[j], k0 + half * GS::KE, k, wf[j]);
    };

    f32x16_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // The MFMAs of one slice: A from LDS buffer `buf`, B decoded from wf.  The
    // operands of k step s+1 are read and decoded before the MFMAs of step s.
    auto mfma_slice = [&](int buf, const Frag (&wf)[TJ]) {
        const uint16_t* as = xs_lds + buf * kXTileElems + (wm * 32 * TI + l32) * kXStride + half * GS::KE;
        bf16x8_t a[2][TI], b[2][TJ];
        auto operands = [&](auto step, bf16x8_t(&ao)[TI], bf16x8_t(&bo)[TJ], const Frag (&wd)[TJ]) {
            constexpr int S = decltype(step)::value;
#pragma unroll
            for (int i = 0; i < TI; ++i) ao[i] = *reinterpret_cast<const bf16x8_t*>(as + i * 32 * kXStride + S * 8);
#pragma unroll
            for (int j = 0; j < TJ; ++j) bo[j] = decode_step<FMT, S>(wd[j]);
        };
        auto mfmas = [&](const bf16x8_t(&ao)[TI], const bf16x8_t(&bo)[TJ]) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao[i], bo[j], acc[i][j], 0, 0, 0);
        };
        // MXFP8 (block_operand.hpp): fragments with an E8M0 byte below kMx8Lift
        // take part in the main MFMAs with zero codes (one code path for every
        // slice); a wave holding one adds their lifted part afterwards.
        Frag we[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            we[j] = wf[j];
            if constexpr (FMT == kMXFP8) {
                const bool lo = frag_lifted(wf[j]);
#pragma unroll
                for (int d = 0; d < Frag::DW; ++d) we[j].w[d] = lo ? 0u : wf[j].w[d];
            }
        }
        if constexpr (GS::STEPS == 4) {
            operands(std::integral_constant<int, 0>{}, a[0], b[0], we);
            operands(std::integral_constant<int, 1>{}, a[1], b[1], we);
            mfmas(a[0], b[0]);
            operands(std::integral_constant<int, 2>{}, a[0], b[0], we);
            mfmas(a[1], b[1]);
            operands(std::integral_constant<int, 3>{}, a[1], b[1], we);
            mfmas(a[0], b[0]);
            mfmas(a[1], b[1]);
        } else {
            operands(std::integral_constant<int, 0>{}, a[0], b[0], we);
            operands(std::integral_constant<int, 1>{}, a[1], b[1], we);
            mfmas(a[0], b[0]);
            mfmas(a[1], b[1]);
        }
        if constexpr (FMT == kMXFP8) {
            bool lo = false;
#pragma unroll
            for (int j = 0; j < TJ; ++j) lo = lo || frag_lifted(wf[j]);
            if (__ballot(lo) != 0) {
                // lifted part (decoded 2^3 larger): the accumulators are scaled by 2^3
                // around its MFMAs, so it accumulates in place (scaling by a power of
                // two commutes with fp32 rounding away from overflow and subnormals)
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j) acc[i][j] *= 1.0f / kMx8Unlift;
                static_for<0, GS::STEPS>([&](auto step) {
                    constexpr int S = decltype(step)::value;
#pragma unroll
                    for (int i = 0; i < TI; ++i)
                        a[0][i] = *reinterpret_cast<const bf16x8_t*>(as + i * 32 * kXStride + S * 8);
#pragma unroll
                    for (int j = 0; j < TJ; ++j) b[0][j] = decode_step_part<FMT, S, true>(wf[j]);
                    mfmas(a[0], b[0]);
                });
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j) acc[i][j] *= kMx8Unlift;
            }
        }
    };

    // Slice s uses LDS buffer s & 1 and W set s & 1 (wa even, wb odd).  Loads
    // past the last slice re-read the last one (cache hits), so no load sits
    // in a branch.
    const int64_t nk = (k + kBK - 1) / kBK;
    const int64_t klast = (nk - 1) * kBK;
    auto kof = [&](int64_t s) { return s < nk ? s * kBK : klast; };
    Frag wa[TJ], wb[TJ];
    load_x(0);
    load_w(0, wa);
    store_x(0);
    load_x(kof(1));
    load_w(kof(1), wb);
    lds_barrier();
    int64_t s = 0;
    for (; s + 1 < nk; s += 2) {
        mfma_slice(0, wa);
        store_x(1);  // slice s+1
        load_x(kof(s + 2));
        load_w(kof(s + 2), wa);
        lds_barrier();
        mfma_slice(1, wb);
        store_x(0);  // slice s+2
        load_x(kof(s + 3));
        load_w(kof(s + 3), wb);
        lds_barrier();
    }
    if (s < nk) mfma_slice(0, wa);

    // Output: lane (half, l32) of fragment (i, j) holds rows 8r + 4*half + q
    // (element 4r + q) of column l32.  Full tiles store without bounds checks.
    const float g = (FMT == kNVFP4) ? gscale[0] : 1.0f;
    const int64_t rbase = m0 + wm * 32 * TI + half * 4, cbase = n0 + wn * 32 * TJ + l32;
    const bool full = (m0 + BM <= m) && (n0 + BN <= nend);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int64_t col = cbase + j * 32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = rbase + i * 32 + (e >> 2) * 8 + (e & 3);
                if (!full && (row >= m || col >= nend)) continue;
                const float v = acc[i][j][e] * g;
                if (y_bf16) reinterpret_cast<uint16_t*>(yv)[row * n + col] = f32_to_bf16_rne(v);
                else reinterpret_cast<float*>(yv)[row * n + col] = v;
            }
        }
}

// One launch over output columns noff .. noff + ncols - 1 with tiles of
// (64 TI) x (128 TJ).
template <int FMT, bool ROW8, int TI, int TJ>
static void launch_gemm_part(const GemmArgs& a, int64_t noff, int64_t ncols, hipStream_t st) {
    constexpr int BM = 64 * TI, BN = 128 * TJ;
    const int64_t tiles = ((a.m + BM - 1) / BM) * ((ncols + BN - 1) / BN);
    // The XCD-aware order needs the tile count to be a multiple of 8 (each
    // XCD then owns exactly tiles/8 consecutive tiles); otherwise plain order.
    const int xcd_order = (tiles % 8 == 0) ? 1 : 0;
    const size_t lds = (size_t)2 * GemmSlice<FMT, BM>::XTILE * sizeof(uint16_t);
    hipLaunchKernelGGL((gemm_kernel<FMT, ROW8, TI, TJ>), dim3((unsigned)tiles), dim3(kGemmThreads), lds, st, a.codes,
                       a.scales, a.gscale, a.x, a.y, a.y_bf16, a.m, a.n, a.k, xcd_order, noff, ncols);
}

// 256 x 256 tiles, as many workgroups at once as fit on the device (one per
// CU).  When the tile count leaves a last, partly filled round (4096 x 25600:
// 1600 tiles, 256 at once), the last tile columns that make up that round go to
// a second launch of 128 x 128 tiles, which spreads them over every CU (MI355X,
// 4096 x 25600 x 5120 MXFP4: 1278 -> 1243 us; those 64 tiles took 136 us as a
// partial round of 256 x 256 tiles, 105 us as 128 x 128 tiles, 148 us as
// 64 x 128 tiles; a full round takes 188 us).
template <int FMT, bool ROW8>
static void launch_gemm_rows(const GemmArgs& a, hipStream_t st) {
    static std::atomic<int> per_cu_cache{-1};
    int per_cu = per_cu_cache.load(std::memory_order_relaxed);
    if (per_cu < 0) {
        const size_t lds = (size_t)2 * GemmSlice<FMT>::XTILE * sizeof(uint16_t);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_kernel<FMT, ROW8, 4, 2>, kGemmThreads, lds) !=
                hipSuccess || per_cu < 1) {
            (void)hipGetLastError();
            per_cu = 1;
        }
        per_cu_cache.store(per_cu, std::memory_order_relaxed);
    }
    const int64_t slots = (int64_t)a.cus * per_cu;
    const int64_t mt = (a.m + kBM - 1) / kBM, nt = (a.n + kBN - 1) / kBN;
    int64_t tail = 0;  // tile columns for the second launch
    if (mt * nt > slots && (mt * nt) % slots != 0)
        for (int64_t c = 1; c <= nt / 8; ++c)
            if (((nt - c) * mt) % slots == 0) {
                tail = c;
                break;
            }
    if (tail == 0) {
        launch_gemm_part<FMT, ROW8, 4, 2>(a, 0, a.n, st);
        return;
    }
    const int64_t n1 = (nt - tail) * kBN;
    launch_gemm_part<FMT, ROW8, 4, 2>(a, 0, n1, st);
    launch_gemm_part<FMT, ROW8, 2, 1>(a, n1, a.n - n1, st);
}

template <int FMT>
static void launch_gemm_inst(const GemmArgs& a, hipStream_t st) {
    // NVFP4 rows of an odd multiple of 16 elements: 8-byte rows (ROW8)
    if (FMT == kNVFP4 && a.k % 32 != 0) launch_gemm_rows<FMT, FMT == kNVFP4>(a, st);
    else launch_gemm_rows<FMT, false>(a, st);
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
