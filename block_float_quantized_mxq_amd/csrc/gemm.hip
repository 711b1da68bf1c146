// gemm.hip -- prefill GEMM on block-float weights: Y[m][i] = sum_k X[m][k] * W[i][k].
//
// Prefill is compute bound ("The memory wall" section of the "MLxcel 0.8
// release" post, slide 15 of the talk); the pages' fast path decodes the
// quantized weights on the GPU and feeds the matrix unit ("Decoding block-float
// formats in software", slide 12).  Here:
//
//  * A workgroup (4 waves, 2 x 2) owns a 256 x 256 tile of Y; each wave owns
//    128 x 128 = 4 x 4 bf16 MFMA 32x32x16 tiles with fp32 accumulators.
//  * Per 64-wide k slice the workgroup stages X (bf16) and the decoded W slice
//    (bf16, block scale folded in: exact for weights in the normal range) in
//    LDS.  LDS is double buffered and slices are fetched two ahead: the global
//    loads of slice i+2 are issued before the MFMAs of slice i, slice i+1
//    (already in registers) goes to the other buffer after them, and there is
//    one barrier per slice.
//  * Rows of the LDS tiles are padded by 16 bytes so that the MFMA operand
//    reads (32 rows x 16 bytes per lane group) hit distinct banks.
//  * Tiles are ordered so that the 32 workgroups resident on one XCD (the
//    dispatcher deals workgroup i to XCD i mod 8) work on a compact block of
//    4 x 8 tiles and share its X and W slices in that XCD's L2.
//  * The NVFP4 per-tensor scale multiplies the fp32 result; the bf16 output is
//    rounded to nearest even from that fp32 value.
#include <cstdlib>

#include "kernels.hpp"
#include "mxq_device.hpp"

namespace mxq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4g_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256;
constexpr int kGemmThreads = 256;
// LDS row stride (bf16 elements) for a BK-wide slice: 16 bytes of padding.
template <int BK> struct GemmTile {
    static constexpr int STRIDE = BK + 8;
    static constexpr int ELEMS = kBM * STRIDE;  // per operand, per buffer
};

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

// Raw code bytes of 32 consecutive elements of one weight row (16 bytes for
// E2M1, 32 for E4M3) and their scale bytes; elements past k read as zero.
template <int FMT>
struct WPiece {
    static constexpr int DW = (FMT == kMXFP8) ? 8 : 4;
    uint32_t w[DW];
    uint32_t s;  // scale byte(s): one E8M0, or two E4M3 (NVFP4) in bits 7:0 and 15:8
};

template <int FMT>
__device__ __forceinline__ void load_wpiece(const uint8_t* crow, const uint8_t* srow, int64_t k0, int64_t k,
                                            WPiece<FMT>& p) {
    if (k0 >= k) {
#pragma unroll
        for (int i = 0; i < WPiece<FMT>::DW; ++i) p.w[i] = 0u;
        p.s = FMT == kNVFP4 ? 0u : 127u;
        return;
    }
    if constexpr (FMT == kMXFP8) {
        const u32x4g_t* q = reinterpret_cast<const u32x4g_t*>(crow + k0);
        const u32x4g_t v0 = q[0], v1 = q[1];
        p.w[0] = v0[0]; p.w[1] = v0[1]; p.w[2] = v0[2]; p.w[3] = v0[3];
        p.w[4] = v1[0]; p.w[5] = v1[1]; p.w[6] = v1[2]; p.w[7] = v1[3];
        p.s = srow[k0 / 32];
    } else {
        const u32x4g_t v = *reinterpret_cast<const u32x4g_t*>(crow + k0 / 2);
        p.w[0] = v[0]; p.w[1] = v[1]; p.w[2] = v[2]; p.w[3] = v[3];
        if constexpr (FMT == kMXFP4) p.s = srow[k0 / 32];
        else p.s = (uint32_t)srow[k0 / 16] | ((uint32_t)srow[k0 / 16 + 1] << 8);
    }
}

// Decode a piece to 16 dwords of bf16 pairs (element order preserved).
template <int FMT>
__device__ __forceinline__ void decode_wpiece(const WPiece<FMT>& p, uint32_t (&out)[16]) {
    if constexpr (FMT == kMXFP8) {
        // E8M0 scales are powers of two: the conversion applies them exactly.
        const float s = e8m0_to_f32(p.s);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            out[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p.w[d], s, false));
            out[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p.w[d], s, true));
        }
    } else if constexpr (FMT == kMXFP4) {
        const float s = e8m0_to_f32(p.s);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            out[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p.w[d], s, 0));
            out[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p.w[d], s, 1));
            out[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p.w[d], s, 2));
            out[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p.w[d], s, 3));
        }
    } else {
        // The conversion instruction uses only the exponent of its scale operand,
        // so E4M3 block scales (which carry mantissa bits) are applied in fp32:
        // q * s has at most 6 significant bits, so the bf16 result is exact.
        const float s0 = e4m3_to_f32(p.s & 0xFFu);
        const float s1 = e4m3_to_f32((p.s >> 8) & 0xFFu);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float s = d < 2 ? s0 : s1;
            out[4 * d + 0] = scaled_fp4x2_to_bf16x2<0>(p.w[d], s);
            out[4 * d + 1] = scaled_fp4x2_to_bf16x2<1>(p.w[d], s);
            out[4 * d + 2] = scaled_fp4x2_to_bf16x2<2>(p.w[d], s);
            out[4 * d + 3] = scaled_fp4x2_to_bf16x2<3>(p.w[d], s);
        }
    }
}

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

template <int FMT, int BK>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gscale,
                                                            const uint16_t* __restrict__ x, void* __restrict__ yv,
                                                            int y_bf16, int64_t m, int64_t n, int64_t k,
                                                            int xcd_order) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [2 buffers][A, B][ELEMS]
    constexpr int kLdsStride = GemmTile<BK>::STRIDE, kTileElems = GemmTile<BK>::ELEMS;
    constexpr int XR = BK / 8;          // threads per X row slice (16 bytes each)
    constexpr int XROWS = 256 / XR;     // X rows per load round
    constexpr int XRND = kBM / XROWS;   // load rounds per slice
    constexpr int WP = BK / 32;         // 32-element W pieces per thread per slice

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t mt = (m + kBM - 1) / kBM, nt = (n + kBN - 1) / kBN;
    int64_t tm, tn;
    if (xcd_order) tile_of(blockIdx.x, mt, nt, tm, tn);
    else { tm = blockIdx.x / nt; tn = blockIdx.x % nt; }
    const int64_t m0 = tm * kBM, n0 = tn * kBN;

    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t sbytes = k / block_elems(FMT);

    // X loader: XRND rounds of XROWS rows; XR consecutive lanes cover one row's
    // BK-wide slice (16 bytes each).
    const int xr = tid / XR, xq = tid % XR;
    const uint16_t* xrow[XRND];
#pragma unroll
    for (int i = 0; i < XRND; ++i) {
        int64_t r = m0 + i * XROWS + xr;
        r = r < m ? r : m - 1;
        xrow[i] = x + r * k + xq * 8;
    }
    // W loader: thread -> (row tid, the slice's 32-element pieces).
    int64_t wr = n0 + tid;
    wr = wr < n ? wr : n - 1;
    const uint8_t* crow = codes + wr * rowbytes;
    const uint8_t* srow = scales + wr * sbytes;

    // Two register sets hold slices in flight: slice s lives in set s & 1.
    u32x4g_t xa[2][XRND];
    WPiece<FMT> wp[2][WP];
    auto load_slice = [&](int set, int64_t kt) {
#pragma unroll
        for (int i = 0; i < XRND; ++i) {
            if (kt + xq * 8 < k) xa[set][i] = *reinterpret_cast<const u32x4g_t*>(xrow[i] + kt);
            else xa[set][i] = u32x4g_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int h = 0; h < WP; ++h) load_wpiece<FMT>(crow, srow, kt + 32 * h, k, wp[set][h]);
    };
    auto store_slice = [&](int set, int buf) {
        uint16_t* As = lds + (2 * buf) * kTileElems;
        uint16_t* Bs = lds + (2 * buf + 1) * kTileElems;
#pragma unroll
        for (int i = 0; i < XRND; ++i)
            *reinterpret_cast<u32x4g_t*>(As + (i * XROWS + xr) * kLdsStride + xq * 8) = xa[set][i];
#pragma unroll
        for (int h = 0; h < WP; ++h) {
            uint32_t d[16];
            decode_wpiece<FMT>(wp[set][h], d);
            u32x4g_t* bd = reinterpret_cast<u32x4g_t*>(Bs + tid * kLdsStride + h * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q) bd[q] = u32x4g_t{d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]};
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // MFMAs of one slice.  Operand fragments are double buffered in registers:
    // the LDS reads of step ks+1 are issued before the 16 MFMAs of step ks and
    // interleaved with them (scheduling groups: one MFMA, one LDS read), so the
    // matrix core does not wait on LDS latency.
    auto read_frags = [&](const uint16_t* As, const uint16_t* Bs, int ks, bf16x8_t (&af)[4], bf16x8_t (&bfr)[4]) {
        const int kk = ks * 16 + (lane >> 5) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 128 + i * 32 + (lane & 31)) * kLdsStride + kk);
            bfr[i] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 128 + i * 32 + (lane & 31)) * kLdsStride + kk);
        }
    };
    auto mfma_slice = [&](int buf) {
        const uint16_t* As = lds + (2 * buf) * kTileElems;
        const uint16_t* Bs = lds + (2 * buf + 1) * kTileElems;
        bf16x8_t af[2][4], bfr[2][4];
        read_frags(As, Bs, 0, af[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK / 16) read_frags(As, Bs, ks + 1, af[cur ^ 1], bfr[cur ^ 1]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
            if (ks + 1 < BK / 16) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
        }
    };

    // Slices are fetched two ahead: while slice it is multiplied out of LDS
    // buffer it & 1, slice it+1 waits in registers (written to the other
    // buffer after the MFMAs) and slice it+2 is on its way from memory.
    const int64_t nk = (k + BK - 1) / BK;
    load_slice(0, 0);
    if (nk > 1) load_slice(1, BK);
    store_slice(0, 0);
    __syncthreads();
    for (int64_t it = 0; it < nk; it += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // h == (it + h) & 1
            const int64_t cur = it + h;
            if (cur < nk) {
                if (cur + 2 < nk) load_slice(h, (cur + 2) * BK);  // set h held slice cur, already in LDS
                mfma_slice(h);
                if (cur + 1 < nk) store_slice(h ^ 1, h ^ 1);
                __syncthreads();
            }
        }
    }

    const float g = (FMT == kNVFP4) ? gscale[0] : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
                if (row >= m) continue;
                const float v = acc[i][j][e] * g;
                if (y_bf16) reinterpret_cast<uint16_t*>(yv)[row * n + col] = f32_to_bf16_rne(v);
                else reinterpret_cast<float*>(yv)[row * n + col] = v;
            }
        }
}

template <int FMT, int BK>
static void launch_gemm_bk(const GemmArgs& a, hipStream_t st) {
    const int64_t mt = (a.m + kBM - 1) / kBM, nt = (a.n + kBN - 1) / kBN;
    const int64_t tiles = mt * nt;
    // The XCD-aware order needs the tile count to be a multiple of 8 (each
    // XCD then owns exactly tiles/8 consecutive tiles); otherwise plain order.
    const int xcd_order = (tiles % 8 == 0) ? 1 : 0;
    const size_t lds = (size_t)4 * GemmTile<BK>::ELEMS * sizeof(uint16_t);
    hipLaunchKernelGGL((gemm_kernel<FMT, BK>), dim3((unsigned)tiles), dim3(kGemmThreads), lds, st, a.codes,
                       a.scales, a.gscale, a.x, a.y, a.y_bf16, a.m, a.n, a.k, xcd_order);
}

// k slice width 64 (144 KB of double-buffered LDS tiles).  Each wave holds a
// 128 x 128 accumulator block in AGPRs, so one wave runs per SIMD whatever the
// LDS size, and the wider slice halves the barriers per k step; measured on
// MI355X it is the faster choice.  MXQ_GEMM_BK=32 selects the 80 KB variant
// (used only to compare variants).
template <int FMT>
static void launch_gemm_inst(const GemmArgs& a, hipStream_t st) {
    const char* env = std::getenv("MXQ_GEMM_BK");
    if (env && std::atoi(env) == 32) launch_gemm_bk<FMT, 32>(a, st);
    else launch_gemm_bk<FMT, 64>(a, st);
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
