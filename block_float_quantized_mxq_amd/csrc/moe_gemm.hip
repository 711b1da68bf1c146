// moe_gemm.hip -- expert-batched MoE GEMM (prefill):
//   y[q][i] = sum_k W[ids[q]][i][k] * x[q / xdiv][k],  q = token * topk + slot
//
// The "Decoding block-float formats in software" section of the "MLxcel 0.8
// release" post credits its MXFP4 MoE prefill gain to kernels that work expert
// by expert.  Kernels:
//
//  * moe_gemm_stream_kernel (rows of whole 32-element blocks, every format):
//    each workgroup finds its expert's pairs in the ids itself (in pair order)
//    and streams the expert's weight rows through registers slice by slice
//    against the pairs' inputs gathered into LDS (below).
//  * moe_group_kernel groups the pairs by expert (counts, prefix sums, and a
//    permutation of the pairs) in a caller workspace, on the GPU, so nothing
//    waits for the host; the register-resident kernel reads it.
//  * moe_gemm_kernel (NVFP4 rows of an odd number of 16-element blocks, whose
//    8-byte rows the streaming kernel's 16-byte loads do not fit): grid (row
//    tile, expert).  Each wave loads its 16 weight
//    rows (over its k range) into registers once; the workgroup then walks
//    the expert's pairs in blocks of 16, gathers their input rows into LDS and
//    runs 16 x 16 x 32 bf16 MFMAs with the 16 pairs as the B operand's columns
//    (the operand layout of gemv_mfma.hpp).  A prompt routes a few dozen
//    pairs to each expert, too few for a GEMM tile of hundreds of rows; here
//    every weight byte is read from HBM once and decoded once per 16 pairs.
//
// The grouping kernel orders an expert's pairs by atomic increments, the
// streaming kernel by pair index; each output value is computed by the same
// arithmetic wherever its pair sits in a block, so results are identical run
// to run.  A pair whose id is outside [0, E) gets
// a NaN output row.
#include "block_operand.hpp"
#include "gemv_mfma.hpp"
#include "kernels.hpp"
#include "rows_core.hpp"

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
// workgroup per CU).
template <int FMT, int MB>
constexpr bool moe_gemm_x_first() { return !(FMT == kNVFP4 && MB == 8); }

template <int FMT, int KS, int MB, bool ROW8>
__global__ __launch_bounds__(kMoeGemmWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void moe_gemm_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ gscale,
    const int32_t* __restrict__ goff, const int32_t* __restrict__ gperm, const uint16_t* __restrict__ x,
    int64_t xdiv, void* __restrict__ yv, int y_bf16, int64_t n, int64_t k) {
    static_assert(FMT == kNVFP4, "E2M1 codes with E4M3 block scales (every other row streams)");
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
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 0>(w[j]), __builtin_bit_cast(bf16x8_t, v[0]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 1>(w[j]), __builtin_bit_cast(bf16x8_t, v[1]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 2>(w[j]), __builtin_bit_cast(bf16x8_t, v[2]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_step<FMT, 3>(w[j]), __builtin_bit_cast(bf16x8_t, v[3]), acc, 0, 0, 0);
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

// ---- streaming variant (E2M1 codes, whole 32-element blocks) -------------------------
//
// Grid (tile of 256 weight rows, expert).  Wave w owns weight rows tile*256 +
// 32w .. +31, one 32-row block of 32x32x16 bf16 MFMAs (the B operand's
// columns); the expert's pairs are taken 64 at a time, two 32-pair blocks as
// the A operand's rows.  Per k slice (64 wide, 32 for E4M3) the workgroup
// gathers the 64 pairs' inputs into LDS (double buffered; one 16- or 8-byte
// piece per thread) and every wave multiplies them with its rows' codes,
// decoded to bf16 in registers; lane (l32, h) holds the 16 bytes of codes of
// half h of the slice of its row l32 (the k order of gemm.hip).  Codes and gathered inputs stream through
// rings of slices in registers, each slot refilled as soon as it is used, so
// a wave keeps loads in flight from start to end, as the GEMV engine does; the register-resident kernel above instead
// loads its whole tile first and then computes, and two such workgroups per
// CU leave HBM idle while both compute.
typedef float f32x16m_t __attribute__((ext_vector_type(16)));
// Slices in flight: kMgDepthW of codes per lane, kMgDepthX of gathered inputs
// per thread (kMgDepthW divides kMgDepthX, the loop's unroll).  MI355X,
// 30B-A3B banks, 512 tokens x top-8, MXFP4 gate/up / down: 92 / 53 us with two
// of each (NVFP4 110 / 59); inputs four ahead 92 / 53 (NVFP4 115 / 59); with
// inputs one ahead, and before the loop's branches and full waits went, 129 / 55.
constexpr int kMgRows = 256, kMgPairs = 64, kMgDepthW = 2, kMgDepthX = 2;
static_assert(kMgDepthX % kMgDepthW == 0, "the unrolled loop indexes both rings statically");
// Slice shape: 64 k (each lane's share of a row one 32-element block, 16 bytes of
// E2M1 codes), or 32 k for E4M3 (a 16-element half block, 16 bytes, as gemm.hip).
template <int FMT>
struct MgSlice {
    static constexpr int BK = FMT == kMXFP8 ? 32 : 64;
    static constexpr int KE = BK / 2;     // k per lane and slice
    static constexpr int STEPS = BK / 16; // MFMA k steps per slice
    static constexpr int XS = BK + 8;     // bf16 per LDS row (16-byte pad: 16 rows' reads hit distinct banks)
    static constexpr int EPT = BK / 8;    // gathered input elements per thread and slice (64 pairs, 512 threads)
};

template <int FMT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void moe_gemm_stream_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ gscale,
    const int32_t* __restrict__ ids, int64_t pairs, int64_t experts, const uint16_t* __restrict__ x,
    int64_t xdiv, void* __restrict__ yv, int y_bf16, int64_t n, int64_t k) {
    using MS = MgSlice<FMT>;
    constexpr int kMgBK = MS::BK, kMgXStride = MS::XS, KE = MS::KE, EPT = MS::EPT;
    using XPiece = std::conditional_t<EPT == 8, u32x4g_t, u32x2g_t>;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kMgPairs * kMgXStride];
    __shared__ int64_t xrow[kMgPairs];  // input row of each pair of the pass, -1 past its end
    __shared__ int64_t qid[kMgPairs];   // output row (pair index) of each pair of the pass
    __shared__ int32_t wcnt[8];         // matches per wave in the chunk being scanned
    __shared__ int64_t s_next;          // where the next pass's scan starts, when a chunk overflows the pass

    // Workgroups are dealt to the 8 XCDs in turn by linear id; when the experts
    // divide evenly, all tiles of an expert go to one XCD so that its pairs'
    // inputs are fetched into one L2.
    int64_t e = blockIdx.y, tile = blockIdx.x;
    if (experts % 8 == 0) {
        const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        const int64_t j = lin / 8;
        e = lin % 8 + 8 * (j / gridDim.x);
        tile = j % gridDim.x;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t sbytes = k / block_elems(FMT);
    const int64_t r0 = tile * kMgRows + wave * 32;
    const int64_t wrow = r0 + l32 < n ? r0 + l32 : n - 1;
    const uint8_t* crow = codes + (e * n + wrow) * rowbytes;
    const uint8_t* srow = scales + (e * n + wrow) * sbytes;
    const float gmul = (FMT == kNVFP4) ? gscale[e] : 1.0f;
    const int64_t nk = (k + kMgBK - 1) / kMgBK;
    const int gp = tid >> 3, gc = tid & 7;  // gather: pair gp, columns EPT gc .. EPT gc + EPT - 1 of the slice
    const uint64_t below = (uint64_t(1) << lane) - 1;

    // The expert's pairs, in pair order, 64 per pass, found by scanning the ids
    // (no separate grouping launch): each thread loads 8 ids at once, chunk j of
    // 512 consecutive pairs is compacted by wave ballots and a per-wave prefix.
    // The scan resumes where the previous pass stopped.  Workgroups of expert 0
    // also write NaN to their 256 columns of every pair with an invalid id.
    constexpr int kScanIds = 8;
    int64_t pos = 0;  // workgroup uniform
    using Frag = WFrag<FMT, KE>;
    // this lane's block of slice s (cached loads: the other blocks of each 128-byte
    // line come with the next slices); past k, zero codes and a unit scale are
    // selected when the block is decoded
    auto load_w = [&](int64_t s, Frag& f) {
        const int64_t kb = s * kMgBK + half * KE;
        const int64_t kc = kb < k ? kb : 0;
        const u32x4g_t v = *reinterpret_cast<const u32x4g_t*>(crow + (FMT == kMXFP8 ? kc : kc / 2));
#pragma unroll
        for (int d = 0; d < 4; ++d) f.w[d] = v[d];
        if constexpr (FMT == kNVFP4) f.s = (uint32_t)srow[kc / 16] | ((uint32_t)srow[kc / 16 + 1] << 8);
        else f.s = srow[kc / 32];
    };
    auto live = [&](int64_t s, const Frag& f) {
        const bool ok = s * kMgBK + half * KE < k;
        Frag g;
#pragma unroll
        for (int d = 0; d < 4; ++d) g.w[d] = ok ? f.w[d] : 0u;
        g.s = ok ? f.s : (FMT == kNVFP4 ? 0x3838u : 127u);
        return g;
    };
    for (;;) {
        // the first slices' codes are requested before the scan (they do not depend on it)
        Frag ring[kMgDepthW];
        static_for<0, kMgDepthW>([&](auto J) { load_w(J, ring[J]); });
        __syncthreads();  // the previous pass is done with xrow, qid and xs
        int found = 0;
        while (found < kMgPairs && pos < pairs) {
            int32_t id[kScanIds];
#pragma unroll
            for (int j = 0; j < kScanIds; ++j) {
                const int64_t q = pos + 512 * j + tid;
                id[j] = q < pairs ? ids[q] : (int32_t)experts;  // past the end: matches no expert
            }
            bool full = false;
#pragma unroll
            for (int j = 0; j < kScanIds; ++j) {
                const int64_t q = pos + 512 * j + tid;
                const bool hit = id[j] == (int32_t)e;
                if (e == 0 && q < pairs && (id[j] < 0 || id[j] >= (int32_t)experts)) {
                    for (int c = 0; c < kMgRows; ++c) {
                        const int64_t col = tile * kMgRows + c;
                        if (col < n) {
                            if (y_bf16) reinterpret_cast<uint16_t*>(yv)[q * n + col] = 0x7FC0u;
                            else reinterpret_cast<float*>(yv)[q * n + col] = __builtin_nanf("");
                        }
                    }
                }
                const uint64_t mask = __ballot(hit);
                if (lane == 0) wcnt[wave] = __popcll(mask);
                __syncthreads();
                int base = found, tot = 0;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    base += w < wave ? wcnt[w] : 0;
                    tot += wcnt[w];
                }
                const int idx = base + __popcll(mask & below);
                if (hit && idx < kMgPairs) {
                    qid[idx] = q;
                    xrow[idx] = q / xdiv;
                }
                if (hit && idx == kMgPairs) s_next = q;  // the first pair of the next pass
                __syncthreads();
                if (found + tot >= kMgPairs) {  // the pass is full (uniform)
                    pos = found + tot > kMgPairs ? s_next : pos + 512 * (j + 1);
                    found = kMgPairs;
                    full = true;
                    break;
                }
                found += tot;
            }
            if (!full) pos += 512 * kScanIds;
        }
        if (found == 0) break;
        const int np = found;
        if (tid < kMgPairs && tid >= np) {
            qid[tid] = -1;
            xrow[tid] = -1;
        }
        __syncthreads();
        const int64_t xr = xrow[gp];
        // Loads without branches and without touching their results until needed (a
        // branch around a load, or a select right after it, makes the compiler wait for
        // every load in flight): addresses clamped into the tensors, the values
        // selected away past k or past the pass's pairs only where they are used.
        auto gather = [&](int64_t k0) {
            const int64_t kk = k0 + EPT * gc;
            const bool ok = xr >= 0 && kk < k;
            return *reinterpret_cast<const XPiece*>(x + (ok ? xr * k + kk : 0));
        };
        auto put = [&](int buf, int64_t k0, const XPiece& v) {  // v = gather(k0)
            const bool ok = xr >= 0 && k0 + EPT * gc < k;
            *reinterpret_cast<XPiece*>(&xs[buf][gp * kMgXStride + EPT * gc]) = ok ? v : XPiece{};
        };
        // the rings: slice j's codes in ring[j % kMgDepthW]; its gathered inputs in
        // xq[j % kMgDepthX] until stored to LDS at the end of slice j - 1.  Slices are
        // taken kMgDepthX at a time; those past the last one multiply zeros.
        XPiece xq[kMgDepthX];
        put(0, 0, gather(0));
        static_for<1, kMgDepthX>([&](auto J) { xq[J] = gather((int64_t)J * kMgBK); });
        // barriers wait for LDS traffic only (__syncthreads would also wait for every
        // global load in flight, draining the rings at each slice)
        lds_barrier();
        f32x16m_t acc[2];
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[pb][i] = 0.0f;
        const bool two = np > 32;  // wave uniform
        for (int64_t s0 = 0; s0 < nk; s0 += kMgDepthX) {
            static_for<0, kMgDepthX>([&](auto J) {
                const int64_t s = s0 + J;
                constexpr int JW = decltype(J)::value % kMgDepthW;
                xq[J] = gather((s + kMgDepthX) * kMgBK);
                const uint16_t* as = &xs[s & 1][l32 * kMgXStride + half * KE];
                Frag w = live(s, ring[JW]);
                auto mfmas = [&]() {
                    static_for<0, MS::STEPS>([&](auto S) {
                        const bf16x8_t b = decode_step<FMT, decltype(S)::value>(w);
                        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(as + S * 8);
                        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[0], 0, 0, 0);
                        if (two) {
                            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(as + 32 * kMgXStride + S * 8);
                            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[1], 0, 0, 0);
                        }
                    });
                };
                if constexpr (FMT != kMXFP8) {
                    mfmas();
                } else {
                    // E4M3 blocks with an E8M0 byte below kMx8Lift (rare; the branch is
                    // wave uniform): first the other fragments, then the lifted ones,
                    // decoded 2^kMx8Lift larger, against the inputs scaled by 2^-kMx8Lift
                    // (exact in bf16 down to inputs whose products with such weights lie
                    // below the fp32 subnormals).
                    const bool lifted = __ballot(frag_lifted(w)) != 0;
                    if (lifted) {
                        const bool lo = frag_lifted(w);
#pragma unroll
                        for (int d = 0; d < Frag::DW; ++d) w.w[d] = lo ? 0u : w.w[d];
                    }
                    mfmas();
                    if (lifted) {
                        w = live(s, ring[JW]);
                        const bool lo = frag_lifted(w);
#pragma unroll
                        for (int d = 0; d < Frag::DW; ++d) w.w[d] = lo ? w.w[d] : 0u;
                        w.s = lo ? w.s + kMx8Lift : 127u;
                        // 8 bf16 times 2^-kMx8Lift: the exponent field lowered; inputs below
                        // 2^-123 become zeros of their sign (their products with these weights
                        // are far below the fp32 subnormals), infinities and NaNs stay
                        auto down = [](const uint16_t* p) {
                            const u32x4g_t v = *reinterpret_cast<const u32x4g_t*>(p);
                            u32x4g_t r;
#pragma unroll
                            for (int d = 0; d < 4; ++d) {
                                uint32_t o = 0u;
#pragma unroll
                                for (int hh = 0; hh < 2; ++hh) {
                                    const uint32_t h = (v[d] >> (16 * hh)) & 0xFFFFu;
                                    const uint32_t e = (h >> 7) & 0xFFu;
                                    const uint32_t q = e == 0xFFu ? h : (e > kMx8Lift ? h - (kMx8Lift << 7) : (h & 0x8000u));
                                    o |= q << (16 * hh);
                                }
                                r[d] = o;
                            }
                            return __builtin_bit_cast(bf16x8_t, r);
                        };
                        static_for<0, MS::STEPS>([&](auto S) {
                            const bf16x8_t b = decode_step<FMT, decltype(S)::value>(w);
                            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(down(as + S * 8), b, acc[0], 0, 0, 0);
                            if (two)
                                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(down(as + 32 * kMgXStride + S * 8), b,
                                                                                 acc[1], 0, 0, 0);
                        });
                    }
                }
                load_w(s + kMgDepthW, ring[JW]);
                put((int)((s + 1) & 1), (s + 1) * kMgBK, xq[(decltype(J)::value + 1) % kMgDepthX]);
                lds_barrier();
            });
        }
        // acc[pb] element 4 r + q: pair pb*32 + 8 r + 4 half + q, weight row r0 + l32
        if (r0 + l32 < n) {
#pragma unroll
            for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int p = pb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                    if (p < np) {
                        const float v = acc[pb][i] * gmul;
                        const int64_t o = qid[p] * n + r0 + l32;
                        if (y_bf16) reinterpret_cast<uint16_t*>(yv)[o] = f32_to_bf16_rne(v);
                        else reinterpret_cast<float*>(yv)[o] = v;
                    }
                }
        }
    }
}

template <int FMT>
static void launch_moe_gemm_stream(const MoeGemmArgs& a, hipStream_t st) {
    const int64_t tiles = (a.n + kMgRows - 1) / kMgRows;
    hipLaunchKernelGGL(moe_gemm_stream_kernel<FMT>, dim3((unsigned)tiles, (unsigned)a.experts), dim3(512), 0, st,
                       a.codes, a.scales, a.gscale, a.ids, a.m * a.topk, a.experts, a.x,
                       a.x_per_slot ? (int64_t)1 : a.topk, a.y, a.y_bf16, a.n, a.k);
}

// The register-resident kernel runs NVFP4 rows of an odd number of 16-element
// blocks (8-byte rows); everything else takes the streaming kernel.
template <int FMT, int KS, int MB>
static void launch_moe_gemm_ks(const MoeGemmArgs& a, const int32_t* goff, const int32_t* gperm, hipStream_t st) {
    constexpr int ROWS = kMoeGemmWaves / KS * 16;
    const int64_t tiles = (a.n + ROWS - 1) / ROWS;
    static_assert(kPairsPerBlock == 16, "moe_gemm_x_lds assumes blocks of 16 pairs");
    hipLaunchKernelGGL((moe_gemm_kernel<FMT, KS, MB, FMT == kNVFP4>), dim3((unsigned)tiles, (unsigned)a.experts),
                       dim3(kMoeGemmWaves * 64), (size_t)moe_gemm_x_lds(a.k), st, a.codes, a.scales, a.gscale, goff,
                       gperm, a.x, a.x_per_slot ? (int64_t)1 : a.topk, a.y, a.y_bf16, a.n, a.k);
}

// Streaming kernel: rows of whole 32-element blocks (every MX row; NVFP4 with
// k % 32 == 0).  Register-resident kernel (the other NVFP4 rows), register
// blocks per lane (MB) and k split (KS): the smallest capacity 4 * MB * KS
// blocks that holds the row, at most 8 blocks per lane (MI355X, 30B-A3B gate/up
// bank in MXFP4, 512-token prompt: 2 x 8 148 us, 1 x 16 162 us, 4 x 4 179 us;
// its down bank: 1 x 6 93 us, 2 x 4 129 us).
template <int FMT>
static bool launch_moe_gemm_inst(const MoeGemmArgs& a, hipStream_t st) {
    const int64_t pairs = a.m * a.topk;
    int32_t* goff = a.workspace;
    int32_t* gperm = a.workspace + a.experts + 1;
    auto group = [&]() {
        hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, st, a.ids, pairs, a.experts, goff,
                           gperm, a.y, a.y_bf16, a.n);
    };
    if (a.k % 32 == 0) {
        launch_moe_gemm_stream<FMT>(a, st);
        return true;
    }
    if constexpr (FMT != kNVFP4) {
        return false;  // MX rows are whole 32-element blocks
    } else {
        const int64_t nblk = (a.k + 31) / 32;
        static constexpr int kCand4[][2] = {{1, 4}, {1, 6}, {1, 8}, {2, 6}, {2, 8}, {4, 6}, {4, 8}};
        int best_ks = 0, best_mb = 0;
        int64_t best_cap = 0;
        auto consider = [&](int ks, int mb) {
            const int64_t cap = 4LL * ks * mb;
            if (cap >= nblk && (best_ks == 0 || cap < best_cap)) { best_ks = ks; best_mb = mb; best_cap = cap; }
        };
        for (const auto& c : kCand4) consider(c[0], c[1]);
        if (best_ks == 0) return false;
        group();
#define MXQ_MG_CASE(KS_, MB_) \
    if (best_ks == KS_ && best_mb == MB_) { launch_moe_gemm_ks<FMT, KS_, MB_>(a, goff, gperm, st); return true; }
        MXQ_MG_CASE(1, 4) MXQ_MG_CASE(1, 6) MXQ_MG_CASE(1, 8) MXQ_MG_CASE(2, 6) MXQ_MG_CASE(2, 8) MXQ_MG_CASE(4, 6)
        MXQ_MG_CASE(4, 8)
#undef MXQ_MG_CASE
        return false;
    }
}

bool launch_moe_gemm(const MoeGemmArgs& a, hipStream_t st) {
    if (a.experts > kMaxGroupExperts) return false;
    if (a.k % 32 != 0 && moe_gemm_x_lds(a.k) > kMoeGemmMaxXLds) return false;  // (the staging kernel's LDS)
    switch (a.fmt) {
        case kMXFP4: return launch_moe_gemm_inst<kMXFP4>(a, st);
        case kMXFP8: return launch_moe_gemm_inst<kMXFP8>(a, st);
        case kNVFP4: return launch_moe_gemm_inst<kNVFP4>(a, st);
    }
    return false;
}

}  // namespace mxq
