// moe_gemm.hip -- expert-batched MoE GEMM (prefill):
//   y[q][i] = sum_k W[ids[q]][i][k] * x[q / xdiv][k],  q = token * topk + slot
//
// The "Decoding block-float formats in software" section of the "MLxcel 0.8
// release" post credits its MXFP4 MoE prefill gain to kernels that work expert
// by expert.  One kernel, moe_gemm_stream_kernel, serves every format and row
// length: each workgroup finds its expert's pairs in the ids itself (in pair
// order) and streams the expert's weight rows through registers slice by slice
// against the pairs' inputs gathered into LDS (below).  A prompt routes a few
// dozen pairs to each expert, too few for a GEMM tile of hundreds of rows; here
// every weight byte is read from HBM once per 64 pairs of its expert.
//
// Each output value is computed by the same arithmetic wherever its pair sits
// in a pass, so results are identical run to run.  A pair whose id is outside
// [0, E) gets a NaN output row.
#include "block_operand.hpp"
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

// ---- the streaming kernel -----------------------------------------------------------
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
// a wave keeps loads in flight from start to end, as the GEMV engine does (a
// kernel that first loaded its whole tile into registers and then computed
// left HBM idle while its two workgroups per CU computed).  NVFP4 rows of an
// odd number of 16-element blocks (ROW8: 8-byte aligned rows) load each
// 16-byte share as two 8-byte halves; the row's last share holds one block.
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

template <int FMT, bool ROW8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void moe_gemm_stream_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ gscale,
    const int32_t* __restrict__ ids, int64_t pairs, int64_t experts, const uint16_t* __restrict__ x,
    int64_t xdiv, void* __restrict__ yv, int y_bf16, int64_t n, int64_t k) {
    static_assert(!ROW8 || FMT == kNVFP4, "only NVFP4 rows can be 8-byte multiples");
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
        if constexpr (ROW8) {
            // two 8-byte halves; a share whose second block lies past the row end
            // reads its first half twice and its first scale twice (selected away
            // where the share is decoded)
            const int64_t hi = kc + 32 <= k ? 8 : 0;
            const u32x2g_t v0 = *reinterpret_cast<const u32x2g_t*>(crow + kc / 2);
            const u32x2g_t v1 = *reinterpret_cast<const u32x2g_t*>(crow + kc / 2 + hi);
            f.w[0] = v0[0];
            f.w[1] = v0[1];
            f.w[2] = v1[0];
            f.w[3] = v1[1];
            f.s = (uint32_t)srow[kc / 16] | ((uint32_t)srow[kc / 16 + hi / 8] << 8);
        } else {
            const u32x4g_t v = *reinterpret_cast<const u32x4g_t*>(crow + (FMT == kMXFP8 ? kc : kc / 2));
#pragma unroll
            for (int d = 0; d < 4; ++d) f.w[d] = v[d];
            if constexpr (FMT == kNVFP4) f.s = (uint32_t)srow[kc / 16] | ((uint32_t)srow[kc / 16 + 1] << 8);
            else f.s = srow[kc / 32];
        }
    };
    auto live = [&](int64_t s, const Frag& f) {
        const int64_t kb = s * kMgBK + half * KE;
        const bool ok = kb < k;
        const bool ok2 = ROW8 ? kb + 32 <= k : ok;  // the share's second 16-element block
        Frag g;
        g.w[0] = ok ? f.w[0] : 0u;
        g.w[1] = ok ? f.w[1] : 0u;
        g.w[2] = ok2 ? f.w[2] : 0u;
        g.w[3] = ok2 ? f.w[3] : 0u;
        if constexpr (FMT == kNVFP4) g.s = (ok ? (f.s & 0xFFu) : 0x38u) | (ok2 ? (f.s & 0xFF00u) : 0x3800u);
        else g.s = ok ? f.s : 127u;
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

template <int FMT, bool ROW8>
static void launch_moe_gemm_stream(const MoeGemmArgs& a, hipStream_t st) {
    const int64_t tiles = (a.n + kMgRows - 1) / kMgRows;
    hipLaunchKernelGGL((moe_gemm_stream_kernel<FMT, ROW8>), dim3((unsigned)tiles, (unsigned)a.experts), dim3(512), 0,
                       st, a.codes, a.scales, a.gscale, a.ids, a.m * a.topk, a.experts, a.x,
                       a.x_per_slot ? (int64_t)1 : a.topk, a.y, a.y_bf16, a.n, a.k);
}

bool launch_moe_gemm(const MoeGemmArgs& a, hipStream_t st) {
    if (a.experts > kMaxGroupExperts) return false;
    switch (a.fmt) {
        case kMXFP4:
            if (a.k % 32 != 0) return false;  // MX rows are whole 32-element blocks
            launch_moe_gemm_stream<kMXFP4, false>(a, st);
            return true;
        case kMXFP8:
            if (a.k % 32 != 0) return false;
            launch_moe_gemm_stream<kMXFP8, false>(a, st);
            return true;
        case kNVFP4:
            if (a.k % 32 == 0) launch_moe_gemm_stream<kNVFP4, false>(a, st);
            else launch_moe_gemm_stream<kNVFP4, true>(a, st);
            return true;
    }
    return false;
}

}  // namespace mxq
