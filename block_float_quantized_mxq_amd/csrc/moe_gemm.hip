// moe_gemm.hip -- expert-batched MoE GEMM (prefill):
//   y[q][i] = sum_k W[ids[q]][i][k] * x[q / xdiv][k],  q = token * topk + slot
//
// The "Decoding block-float formats in software" section of the "MLxcel 0.8
// release" post credits its MXFP4 MoE prefill gain to kernels that work expert
// by expert.  Two kernels:
//
//  * moe_group_kernel groups the pairs by expert (counts, prefix sums, and a
//    permutation of the pairs) in a caller workspace, on the GPU, so nothing
//    waits for the host.
//  * moe_gemm_kernel: grid (row tile, expert).  Each wave loads its 16 weight
//    rows (over its k range) into registers once; the workgroup then walks
//    the expert's pairs in blocks of 16, gathers their input rows into LDS and
//    runs 16 x 16 x 32 bf16 MFMAs with the 16 pairs as the B operand's columns
//    (the operand layout of gemv_mfma.hpp).  A prompt routes a few dozen
//    pairs to each expert, too few for a GEMM tile of hundreds of rows; here
//    every weight byte is read from HBM once and decoded once per 16 pairs.
//
// The order of pairs inside a group follows atomic increments; each output
// value is computed by the same arithmetic wherever its pair sits in a block,
// so results are identical run to run.  A pair whose id is outside [0, E) gets
// a NaN output row.
#include "block_operand.hpp"
#include "gemv_mfma.hpp"
#include "kernels.hpp"

namespace mxq {

// ---- grouping ----------------------------------------------------------------------

constexpr int kGroupThreads = 1024;

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(const int32_t* __restrict__ ids, int64_t pairs,
                                                                  int64_t experts, int32_t* __restrict__ goff,
                                                                  int32_t* __restrict__ gperm, void* __restrict__ yv,
                                                                  int y_bf16, int64_t n) {
    __shared__ int cnt[kMaxGroupExperts];
    __shared__ int scan[kGroupThreads];
    const int tid = threadIdx.x;
    const int E = (int)experts;
    for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
    __syncthreads();
    for (int64_t q = tid; q < pairs; q += kGroupThreads) {
        const int e = ids[q];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // inclusive scan of the counts (E <= kGroupThreads) by doubling steps
    int v = tid < E ? cnt[tid] : 0;
    scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < kGroupThreads; off <<= 1) {
        const int add = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        v += add;
        scan[tid] = v;
        __syncthreads();
    }
    if (tid < E) {
        const int start = v - cnt[tid];
        goff[tid] = start;
        cnt[tid] = start;  // running insert position
    }
    if (tid == 0) goff[E] = scan[E - 1];
    __syncthreads();
    for (int64_t q = tid; q < pairs; q += kGroupThreads) {
        const int e = ids[q];
        if (e >= 0 && e < E) {
            gperm[atomicAdd(&cnt[e], 1)] = (int32_t)q;
        } else {
            for (int64_t c = 0; c < n; ++c) {
                if (y_bf16) reinterpret_cast<uint16_t*>(yv)[q * n + c] = 0x7FC0u;
                else reinterpret_cast<float*>(yv)[q * n + c] = __builtin_nanf("");
            }
        }
    }
}

// ---- per-expert matrix-unit product ------------------------------------------------

constexpr int kPairsPerBlock = 16;  // B operand columns
constexpr int kMoeGemmWaves = 8;    // waves per workgroup (measured on MI355X: 8 beat 4 and 16)

// Grid (row tile, expert).  Wave w owns rows tile*ROWS + (w / KS)*16 .. +15 and
// k range w % KS; lane (row l % 16, k group g = l / 16) holds MB whole 32-element
// blocks of its row in registers -- blocks kb0 + 4j + g, j < MB -- loaded once
// and used for every block of 16 pairs, so the expert's weights leave HBM
// once per call.
// XF: the first block's inputs are requested before the weights (below).
// That keeps their registers live across the weight loads; the 4-bit formats
// stay within the 128 registers of two workgroups per CU (their LDS allows
// two) except NVFP4 with eight blocks per lane, which loads its weights first
// (MI355X, 30B-A3B gate/up bank, 512 tokens: 176 us that way, 223 us with one
// workgroup per CU).  E4M3 blocks take twice the registers either way.
template <int FMT, int MB>
constexpr bool moe_gemm_x_first() { return !(FMT == kNVFP4 && MB == 8); }

template <int FMT, int KS, int MB, bool ROW8>
__global__ __launch_bounds__(kMoeGemmWaves * 64) __attribute__((amdgpu_waves_per_eu(FMT == kMXFP8 ? 2 : 4))) void moe_gemm_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ gscale,
    const int32_t* __restrict__ goff, const int32_t* __restrict__ gperm, const uint16_t* __restrict__ x,
    int64_t xdiv, void* __restrict__ yv, int y_bf16, int64_t n, int64_t k) {
    constexpr int NW = kMoeGemmWaves;
    constexpr int ROWS = NW / KS * 16;
    __shared__ __attribute__((aligned(16))) float red[KS > 1 ? NW * 256 : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];  // [16][k + 8] bf16
    __shared__ int64_t xrow_of[kPairsPerBlock];                     // input row of each pair of the block

    const int64_t e = blockIdx.y;
    const int64_t c0 = goff[e];
    const int64_t cnt = goff[e + 1] - c0;
    if (cnt <= 0) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int l = tid & 63;
    const int lr = l & 15;  // row within the wave's 16; also the pair column of the B operand
    const int g = l >> 4;   // k group
    const int wr = wave / KS, kp = wave % KS;

    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t sbytes = k / block_elems(FMT);
    const int64_t nblk = (k + 31) / 32;  // ROW8 (NVFP4, k an odd multiple of 16): the last block is half
    const int64_t kb0 = (int64_t)kp * MB * 4;
    const int64_t kb1 = kb0 + MB * 4 < nblk ? kb0 + MB * 4 : nblk;
    const int64_t rowt = (int64_t)blockIdx.x * ROWS + (int64_t)wr * 16;
    int64_t row = rowt + lr;
    row = row < n ? row : n - 1;
    const uint8_t* crow = codes + (e * n + row) * rowbytes;
    const uint8_t* srow = scales + (e * n + row) * sbytes;
    const float gmul = (FMT == kNVFP4) ? gscale[e] : 1.0f;

    // Gather of the input rows of a block of pairs into LDS: piece i of the
    // block is row i / pieces, 16-byte column i % pieces; a round issues U
    // pieces per thread (all of a 16 x 2048 block in one round), then stores them.
    constexpr int U = 8, NT = NW * 64;
    const int pieces = (int)(k / 8);
    const int64_t xstride = mfma_x_stride(k);
    u32x4g_t xv[U];
    int dst[U];  // LDS 16-byte slot of each piece
    auto gather_issue = [&](int i0, int total) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * NT < total ? i0 + u * NT : i0;
            const int bi = i / pieces, ci = i - bi * pieces;
            dst[u] = bi * (int)(xstride / 8) + ci;
            xv[u] = *reinterpret_cast<const u32x4g_t*>(x + xrow_of[bi] * k + (int64_t)ci * 8);
        }
    };
    auto gather_store = [&](int i0, int total) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * NT < total) reinterpret_cast<u32x4g_t*>(xlds)[dst[u]] = xv[u];
    };
    // The first block's rows are requested before the weights (XF): the loads
    // complete in order, so storing them to LDS then waits for them alone and
    // the weights arrive while the workgroup stages and synchronises.
    constexpr bool XF = moe_gemm_x_first<FMT, MB>();
    if constexpr (XF) {
        const int batch = (int)(cnt < kPairsPerBlock ? cnt : kPairsPerBlock);
        if (tid < batch) xrow_of[tid] = gperm[c0 + tid] / xdiv;
        __syncthreads();
        if (tid < batch * pieces) gather_issue(tid, batch * pieces);
    }

    // the lane's weight blocks: loaded once; blocks outside the k range read
    // a valid block and are zeroed (codes 0, unit scale)
    WFrag<FMT> w[MB];
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const int64_t b = kb0 + 4 * j + g;
        const bool ok = b < kb1;
        valid |= (ok ? 1u : 0u) << j;
        if constexpr (ROW8) load_wfrag<FMT, 32, true>(crow, srow, (ok ? b : 0) * 32, k, w[j]);
        else load_block<FMT>(crow, srow, ok ? b : 0, w[j]);
    }

    // the rest of the first block's staging
    if constexpr (XF) {
        const int total = (int)(cnt < kPairsPerBlock ? cnt : kPairsPerBlock) * pieces;
        if (tid < total) gather_store(tid, total);
        for (int i0 = tid + U * NT; i0 < total; i0 += U * NT) {
            gather_issue(i0, total);
            gather_store(i0, total);
        }
    }
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const bool ok = (valid >> j) & 1u;
#pragma unroll
        for (int d = 0; d < WFrag<FMT>::DW; ++d) w[j].w[d] = ok ? w[j].w[d] : 0u;
        w[j].s = ok ? w[j].s : (FMT == kNVFP4 ? 0x3838u : 127u);
    }
    // MXFP8 weights with an E8M0 byte below kMx8Lift anywhere in the wave: their
    // lifted part runs as a second pass (block_operand.hpp); uniform over the wave
    bool lifted = false;
    if constexpr (FMT == kMXFP8) {
        bool lo = false;
#pragma unroll
        for (int j = 0; j < MB; ++j) lo = lo || frag_lifted<FMT>(w[j]);
        lifted = __ballot(lo) != 0;
    }

    for (int64_t t0 = 0; t0 < cnt; t0 += kPairsPerBlock) {
        const int batch = (int)(cnt - t0 < kPairsPerBlock ? cnt - t0 : kPairsPerBlock);
        const bool xlive = lr < batch;
        if (t0 > 0 || !XF) {
            const int total = batch * pieces;
            __syncthreads();  // the previous block's LDS reads are done
            if (tid < batch) xrow_of[tid] = gperm[c0 + t0 + tid] / xdiv;
            __syncthreads();
            for (int i0 = tid; i0 < total; i0 += U * NT) {
                gather_issue(i0, total);
                gather_store(i0, total);
            }
        }
        __syncthreads();

        f32x4m_t acc = {0.f, 0.f, 0.f, 0.f};
        const u32x4g_t* xp0 = reinterpret_cast<const u32x4g_t*>(xlds) + ((int64_t)lr * xstride + (kb0 + g) * 32) / 8;
        // B operands of block j (4 x 16 bytes of the pair's input), zero for
        // pairs past the block and blocks outside the k range
        auto read_x = [&](int j, u32x4g_t(&v)[4]) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) v[s4] = u32x4g_t{0u, 0u, 0u, 0u};
            if (xlive && ((valid >> j) & 1u)) {
                // ROW8: the last block is half; its staged row ends at k (no read past it)
                const bool half = ROW8 && (kb0 + 4 * j + g) * 32 + 32 > k;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    if (!(half && s4 >= 2)) v[s4] = xp0[j * 16 + s4];
            }
        };
        u32x4g_t vb[2][4];
        read_x(0, vb[0]);
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            // the reads of block j + 1 are issued before the MFMAs of block j;
            // the empty asm keeps the compiler from hoisting later reads
            // (which would hold every block's operands in registers at once)
            if (j + 1 < MB) read_x(j + 1, vb[(j + 1) & 1]);
            const u32x4g_t(&v)[4] = vb[j & 1];
            if constexpr (FMT == kMXFP8) {
                // one code path: lifted blocks take part with zero codes, and a
                // wave holding one adds their lifted part (a rare second pass)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 0, false>(w[j]), __builtin_bit_cast(bf16x8_t, v[0]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 1, false>(w[j]), __builtin_bit_cast(bf16x8_t, v[1]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 2, false>(w[j]), __builtin_bit_cast(bf16x8_t, v[2]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 3, false>(w[j]), __builtin_bit_cast(bf16x8_t, v[3]), acc, 0, 0, 0);
                if (lifted) {
                    f32x4m_t t = {0.f, 0.f, 0.f, 0.f};
                    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 0, true>(w[j]), __builtin_bit_cast(bf16x8_t, v[0]), t, 0, 0, 0);
                    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 1, true>(w[j]), __builtin_bit_cast(bf16x8_t, v[1]), t, 0, 0, 0);
                    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 2, true>(w[j]), __builtin_bit_cast(bf16x8_t, v[2]), t, 0, 0, 0);
                    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step_part<FMT, 3, true>(w[j]), __builtin_bit_cast(bf16x8_t, v[3]), t, 0, 0, 0);
                    acc += t * kMx8Unlift;
                }
            } else {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 0>(w[j]), __builtin_bit_cast(bf16x8_t, v[0]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 1>(w[j]), __builtin_bit_cast(bf16x8_t, v[1]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 2>(w[j]), __builtin_bit_cast(bf16x8_t, v[2]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 3>(w[j]), __builtin_bit_cast(bf16x8_t, v[3]), acc, 0, 0, 0);
            }
            asm volatile("" ::: "memory");
        }

        // k-split sums in a fixed order, then the block's outputs
        if constexpr (KS > 1) {
            *reinterpret_cast<f32x4m_t*>(red + (wave * 64 + l) * 4) = acc;
            __syncthreads();
            if (kp == 0) {
#pragma unroll
                for (int q = 1; q < KS; ++q) acc += *reinterpret_cast<const f32x4m_t*>(red + ((wave + q) * 64 + l) * 4);
            }
        }
        if (kp == 0 && xlive) {
            const int64_t q = gperm[c0 + t0 + lr];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int64_t r = rowt + 4 * g + ii;
                if (r < n) {
                    const float v = acc[ii] * gmul;
                    if (y_bf16) reinterpret_cast<uint16_t*>(yv)[q * n + r] = f32_to_bf16_rne(v);
                    else reinterpret_cast<float*>(yv)[q * n + r] = v;
                }
            }
        }
    }
}

template <int FMT, int KS, int MB>
static void launch_moe_gemm_ks(const MoeGemmArgs& a, const int32_t* goff, const int32_t* gperm, hipStream_t st) {
    constexpr int ROWS = kMoeGemmWaves / KS * 16;
    const int64_t tiles = (a.n + ROWS - 1) / ROWS;
    static_assert(kPairsPerBlock == 16, "moe_gemm_x_lds assumes blocks of 16 pairs");
    const dim3 grid((unsigned)tiles, (unsigned)a.experts);
    if (FMT == kNVFP4 && a.k % 32 != 0)
        hipLaunchKernelGGL((moe_gemm_kernel<FMT, KS, MB, FMT == kNVFP4>), grid, dim3(kMoeGemmWaves * 64),
                           (size_t)moe_gemm_x_lds(a.k), st, a.codes, a.scales, a.gscale, goff, gperm, a.x,
                           a.x_per_slot ? (int64_t)1 : a.topk, a.y, a.y_bf16, a.n, a.k);
    else
        hipLaunchKernelGGL((moe_gemm_kernel<FMT, KS, MB, false>), grid, dim3(kMoeGemmWaves * 64),
                           (size_t)moe_gemm_x_lds(a.k), st, a.codes, a.scales, a.gscale, goff, gperm, a.x,
                           a.x_per_slot ? (int64_t)1 : a.topk, a.y, a.y_bf16, a.n, a.k);
}

// Register blocks per lane (MB) and k split (KS): the smallest capacity
// 4 * MB * KS blocks that holds the row, at most 8 blocks per lane (MI355X,
// 30B-A3B gate/up bank, 512-token prompt: 2 x 8 148 us, 1 x 16 162 us,
// 4 x 4 179 us; its down bank: 1 x 6 93 us, 2 x 4 129 us).  E4M3 blocks take
// twice the registers: at most 4 per lane (6 or 8 spill), split up to 8 ways.
template <int FMT>
static bool launch_moe_gemm_inst(const MoeGemmArgs& a, hipStream_t st) {
    const int64_t pairs = a.m * a.topk;
    int32_t* goff = a.workspace;
    int32_t* gperm = a.workspace + a.experts + 1;
    const int64_t nblk = (a.k + 31) / 32;
    static constexpr int kCand4[][2] = {{1, 4}, {1, 6}, {1, 8}, {2, 6}, {2, 8}, {4, 6}, {4, 8}};
    static constexpr int kCand8[][2] = {{1, 4}, {2, 4}, {4, 4}, {8, 4}};
    int best_ks = 0, best_mb = 0;
    int64_t best_cap = 0;
    auto consider = [&](int ks, int mb) {
        const int64_t cap = 4LL * ks * mb;
        if (cap >= nblk && (best_ks == 0 || cap < best_cap)) { best_ks = ks; best_mb = mb; best_cap = cap; }
    };
    if constexpr (FMT == kMXFP8) {
        for (const auto& c : kCand8) consider(c[0], c[1]);
    } else {
        for (const auto& c : kCand4) consider(c[0], c[1]);
    }
    if (best_ks == 0) return false;
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, st, a.ids, pairs, a.experts, goff, gperm,
                       a.y, a.y_bf16, a.n);
#define MXQ_MG_CASE(KS_, MB_) \
    if (best_ks == KS_ && best_mb == MB_) { launch_moe_gemm_ks<FMT, KS_, MB_>(a, goff, gperm, st); return true; }
    if constexpr (FMT == kMXFP8) {
        MXQ_MG_CASE(1, 4) MXQ_MG_CASE(2, 4) MXQ_MG_CASE(4, 4) MXQ_MG_CASE(8, 4)
    } else {
        MXQ_MG_CASE(1, 4) MXQ_MG_CASE(1, 6) MXQ_MG_CASE(1, 8) MXQ_MG_CASE(2, 6) MXQ_MG_CASE(2, 8) MXQ_MG_CASE(4, 6)
        MXQ_MG_CASE(4, 8)
    }
#undef MXQ_MG_CASE
    return false;
}

bool launch_moe_gemm(const MoeGemmArgs& a, hipStream_t st) {
    if (a.experts > kMaxGroupExperts) return false;
    if (moe_gemm_x_lds(a.k) > kMoeGemmMaxXLds) return false;
    switch (a.fmt) {
        case kMXFP4: return launch_moe_gemm_inst<kMXFP4>(a, st);
        case kMXFP8: return launch_moe_gemm_inst<kMXFP8>(a, st);
        case kNVFP4: return launch_moe_gemm_inst<kNVFP4>(a, st);
    }
    return false;
}

}  // namespace mxq
