// rows_core.hpp -- the streaming inner loop shared by the dense GEMV and the
// expert-indexed MoE GEMV: a 256-thread workgroup reads a tile of weight rows
// once, decodes the codes in registers, contracts them with up to B bf16
// activation vectors and writes fp32 outputs.
//
// Work split (wave64): the workgroup is cut into groups of G lanes.  S groups
// share a set of R rows and split the row's 16-byte chunks between them; each
// lane walks chunks c = (i*S + s)*G + lane, so a wave's 128-bit load covers
// G*S*16 contiguous bytes of a row.  Every lane keeps R*B fp32 accumulators
// (the activation chunk it loads is reused by all R rows).  At the end the G
// lanes of a group are summed with DPP, and the S groups through LDS, in a
// fixed order: results are bit-identical run to run.
//
// Pipelining: a lane's chunk loads for pass i+1 are issued before the
// arithmetic of pass i, the first pass of a tile is issued before the
// activations are staged (so the two memory latencies overlap), and the last
// pass of a tile issues the first pass of the workgroup's next tile.  LDS is
// synchronised with a barrier that waits for LDS operations only, so
// outstanding weight loads stay in flight across it.
//
// Per 16-byte chunk: MXFP4 = one 32-element block (one E8M0 byte), MXFP8 = half
// a 32-element block, NVFP4 = two 16-element blocks (two E4M3 bytes).  An
// 8-byte chunk is used for NVFP4 rows whose byte length is not a multiple of 16.
// MX block scales are powers of two and go into the scaled conversion itself
// (the decoded bf16 value q * 2^(u-127) is exact at every scale byte, with
// MXFP8 blocks of bytes below kMx8Lift decoded 2^3 larger and scaled back on
// their fp32 partial sum);
// NVFP4's E4M3 block scale multiplies the 16-element block's fp32 partial sum,
// and its per-tensor scale multiplies the final sum.
//
// Activations: each lane needs the activation chunk matching its code chunk
// for every batch entry.  With XL the workgroup first copies x[B][k] into LDS
// (unpadded; the 16-byte pieces of a chunk are XOR-swizzled so that 16 lanes
// reading the same piece of 16 consecutive chunks hit distinct banks) and the
// loop reads it from there; otherwise the loop loads it from global memory
// (L1/L2 resident), once per chunk for all R rows.
#pragma once

#include <type_traits>

#include "mxq_device.hpp"

namespace mxq {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int FMT, int CB>
struct ChunkShape {
    static constexpr int DW = CB / 4;                              // code dwords per chunk
    static constexpr int KPC = (FMT == kMXFP8) ? CB : 2 * CB;      // elements per chunk
    static constexpr int NP = KPC / 2;                             // bf16 pairs per chunk
    static constexpr int BS = BlockSize<FMT>::value;               // elements per scale block
    static constexpr int PPS = (BS / 2 < NP) ? BS / 2 : NP;        // pairs sharing one scale
    static constexpr int NSG = NP / PPS;                           // scales per chunk
    static constexpr int XQ = KPC * 2 / 16;                        // 16-byte activation pieces per chunk
};

// LDS layout of staged activations: batch entry (or slot) b, chunk c, piece q
// (16 bytes) sits at 16-byte slot v * XQ + (q ^ x_swizzle(v)) with the flat
// chunk index v = b * nchunks + c; writers and readers both swizzle by v.  The
// 64 banks of 4 bytes span 16 slots.  16 lanes reading chunks v0 .. v0 + 15
// (any v0) cover every residue of v mod 16: with XQ = 4 lane slots are
// 4*(v & 3) + (q ^ ((v >> 2) & 3)) mod 16, with XQ = 2 they are
// 2*(v & 7) + (q ^ ((v >> 3) & 1)), distinct either way, with no padding.
template <int FMT, int CB>
__host__ __device__ constexpr int x_swizzle(int64_t c) {
    return ChunkShape<FMT, CB>::XQ == 4 ? (int)((c >> 2) & 3) : (ChunkShape<FMT, CB>::XQ == 2 ? (int)((c >> 3) & 1) : 0);
}

// LDS bytes needed to stage x[B][k] (bf16).
template <int FMT, int CB>
__host__ __device__ constexpr int64_t x_lds_bytes(int64_t k, int b) {
    return (int64_t)b * k * 2;
}

// Weight codes are read exactly once per call: load them with the nontemporal
// hint so they do not displace the activations from the caches.
template <int CB>
__device__ __forceinline__ void load_code_chunk(const uint8_t* p, uint32_t (&c)[CB / 4]) {
    if constexpr (CB == 16) {
        u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        c[0] = v[0]; c[1] = v[1]; c[2] = v[2]; c[3] = v[3];
    } else {
        u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        c[0] = v[0]; c[1] = v[1];
    }
}

// Scale bytes are loaded without the hint: consecutive passes read the same
// cache line (16 bytes of it at a time), so it must stay cached between them
// (measured on MI355X: nontemporal scale loads re-fetch and cost ~5%).
__device__ __forceinline__ uint32_t load_scale_byte(const uint8_t* p) { return *p; }

// Raw scale bytes for the NSG scale groups of chunk c of one row.
template <int FMT, int CB>
__device__ __forceinline__ void load_scale_bytes(const uint8_t* srow, int64_t c,
                                                 uint32_t (&sb)[ChunkShape<FMT, CB>::NSG]) {
    using CS = ChunkShape<FMT, CB>;
    if constexpr (FMT == kMXFP4) {
        sb[0] = load_scale_byte(srow + c);
    } else if constexpr (FMT == kMXFP8) {
        sb[0] = load_scale_byte(srow + (c >> 1));
    } else if constexpr (CS::NSG == 2) {
        sb[0] = load_scale_byte(srow + 2 * c);
        sb[1] = load_scale_byte(srow + 2 * c + 1);
    } else {
        sb[0] = load_scale_byte(srow + c);
    }
}

// Scale bytes -> fp32 multipliers (E8M0 for MX formats, E4M3 for NVFP4).
template <int FMT, int CB>
__device__ __forceinline__ void scale_values(const uint32_t (&sb)[ChunkShape<FMT, CB>::NSG],
                                             float (&sc)[ChunkShape<FMT, CB>::NSG]) {
#pragma unroll
    for (int q = 0; q < ChunkShape<FMT, CB>::NSG; ++q)
        sc[q] = (FMT == kNVFP4) ? e4m3_to_f32(sb[q]) : e8m0_to_f32(sb[q]);
}

// Scale multipliers for the NSG scale groups of chunk c of one row.
template <int FMT, int CB>
__device__ __forceinline__ void load_chunk_scales(const uint8_t* srow, int64_t c, float (&sc)[ChunkShape<FMT, CB>::NSG]) {
    uint32_t sb[ChunkShape<FMT, CB>::NSG];
    load_scale_bytes<FMT, CB>(srow, c, sb);
    scale_values<FMT, CB>(sb, sc);
}

// Threads per workgroup of every streaming kernel.
constexpr int kThreads = 256;

template <int G, int S, int R>
struct RowTile {
    static_assert(kThreads % (G * S) == 0, "groups must tile the workgroup");
    static constexpr int GROUPS = kThreads / G;
    static constexpr int ROWSETS = GROUPS / S;
    static constexpr int ROWS = ROWSETS * R;  // rows per workgroup
};

// Copies x[B][k] into LDS (layout above; with MM the flat chunk index is
// v = c * B + b instead, batch entries of one chunk side by side).  Every
// thread of the workgroup must call it; it ends with a barrier.
template <int FMT, int CB, int B, bool MM = false>
__device__ __forceinline__ void stage_x(const uint16_t* const (&xs)[B], int64_t k, uint8_t* xlds) {
    using CS = ChunkShape<FMT, CB>;
    constexpr int U = 8;  // pieces per thread in flight
    const int64_t pieces = k * 2 / 16;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(xs[b]);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(xlds);
        for (int64_t t0 = threadIdx.x; t0 < pieces; t0 += U * kThreads) {
            u32x4_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t t = t0 + (int64_t)u * kThreads;
                if (t < pieces) v[u] = src[t];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t t = t0 + (int64_t)u * kThreads;
                if (t < pieces) {
                    const int64_t c = t / CS::XQ;
                    const int q = (int)(t % CS::XQ);
                    const int64_t v_flat = MM ? c * B + b : (int64_t)b * (pieces / CS::XQ) + c;
                    dst[v_flat * CS::XQ + (q ^ x_swizzle<FMT, CB>(v_flat))] = v[u];
                }
            }
        }
    }
    lds_barrier();
}

// The streaming engine for one workgroup: geometry of the lane's chunks and
// the pipelined pass loop over row tiles.  Every thread of the workgroup must
// take part in every call.
// One pass of one lane: R code chunks and their scale bytes.
template <int FMT, int CB, int R>
struct RowPass {
    uint32_t cw[R][ChunkShape<FMT, CB>::DW];
    uint32_t sb[R][ChunkShape<FMT, CB>::NSG];
};

// Row pointers of one tile for one lane.
template <int R>
struct RowPtrs {
    const uint8_t* c[R];
    const uint8_t* s[R];
};

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (compile-time indices).
template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < E) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, E>(f);
    }
}

// N pass buffers indexed at compile time only (an array indexed by a loop
// counter would live in scratch memory until the loop is unrolled).
template <class P, int N>
struct PassRing {
    P head;
    PassRing<P, N - 1> tail;
    template <int I>
    __device__ __forceinline__ P& at() {
        if constexpr (I == 0) return head;
        else return tail.template at<I - 1>();
    }
};
template <class P>
struct PassRing<P, 0> {};

// Where the next pass to be loaded lies: tile tl of `count` (rows first +
// tl * row_step), pass il, chunk cl, row pointers rl.  Past the last pass it
// points at the first activation vector (a pass reads at most k/2 code bytes
// and k/16 scale bytes of it, both within its 2k bytes), so loads can be
// issued unconditionally and then hit the cache.
template <int R>
struct RowCursor {
    int64_t first, row_step, count, tl, il;
    int cl;
    RowPtrs<R> rl;
    const uint8_t* dummy;
};

// With SLOTS the S groups of a row set do not split one row: group s streams
// all of its own row (the caller points each lane's `codes`/`scales` at its
// group's matrix), against activation vector s of the staged LDS block (B must
// be 1), and the S partial sums are combined with per-group multipliers.
//
// With MM (matrix mode, batch up to 4) the contraction runs on the 16 x 16 x 32
// bf16 MFMA instead of dot2, with the loads of the FMA mode (each wave
// instruction covers 4 rows x 256 contiguous bytes).  Lane l of a wave holds
// chunk position 4 * (l / 16) + l % 4 of row (l / 4) % 4 of each of its R
// four-row groups.  As the A operand, lane l is MFMA row i = l % 16 = 4 * row
// + segment (segment s = l % 4) and k group l / 16, so MFMA row (row, s) sums
// the chunks at positions 4g + s.  The B operand's 16 columns are (activation
// vector v, segment s') = (l / 4 % 4, l % 4): lane l reads vector v at its own
// chunk, the same positions.  The product then holds, for every row and
// vector, the sums of the 4 segments on the diagonal blocks s = s' (the other
// 12 of each 16 are discarded); they are added by one quad reduction at the
// end of the tile.  The vector ALU only decodes, so batch 4 costs what batch 1
// does; S splits k across the waves of the workgroup.
//
// Paired mode (PAIR): the tile's rows are taken in pairs, logical row 2i + h
// being physical row i + h * n/2 (n even), so each lane holds the gate row i
// and the up row i of a SwiGLU layer (gate rows first, up rows second); the
// tile's end stores both products and, to `act`, the activation
// bf16(silu(gate) * up).
template <int FMT, int CB, int B, int G, int S, int R, bool XL, bool SLOTS = false, bool MM = false,
          bool PAIR = false>
struct RowEngine {
    using CS = ChunkShape<FMT, CB>;
    using T = RowTile<G, S, R>;
    using Pass = RowPass<FMT, CB, R>;
    using Rows = RowPtrs<R>;
    using Cursor = RowCursor<R>;
    static_assert(!MM || (G == 16 && B <= 4 && !SLOTS && (S == 1 || S == 2 || S == 4)),
                  "matrix mode: 16 chunk positions, batch <= 4, k split across the 4 waves");
    static_assert(!PAIR || (S == 1 && R % 2 == 0 && !SLOTS && !MM), "paired rows: one k group, rows in pairs");
    static constexpr int NA = MM ? 4 : B;  // accumulators per row (MM: the 4 rows of an MFMA block)
    static constexpr int RED_FLOATS = S > 1 ? S * T::ROWSETS * R * NA : 1;
    static constexpr int WSETS = 4 / S;    // MM: wave row groups per workgroup

    const uint8_t* codes;
    const uint8_t* scales;
    int64_t n, rowbytes, sbytes, nchunks, step, c0, niter;
    int lane, rs, sp, mi;
    // PAIR: output ys[b] = y0 + q n is position q; its activations go to act0 + q n/2
    const float* y0 = nullptr;
    uint16_t* act0 = nullptr;

    __device__ __forceinline__ RowEngine(const uint8_t* codes_, const uint8_t* scales_, int64_t n_, int64_t k) {
        codes = codes_;
        scales = scales_;
        n = n_;
        const int tid = threadIdx.x;
        if constexpr (MM) {
            const int l = tid & 63;
            lane = 4 * (l >> 4) + (l & 3);  // chunk position in the 16-chunk window
            mi = (l >> 2) & 3;              // row within a four-row group; activation vector of the B operand
            rs = (tid >> 6) / S;            // the wave's row group
            sp = (tid >> 6) % S;
        } else {
            lane = tid % G;
            const int gid = tid / G;
            rs = gid / S;
            sp = gid % S;
            mi = 0;
        }
        rowbytes = code_bytes_per_row(FMT, k);
        sbytes = k / CS::BS;
        nchunks = rowbytes / CB;
        step = SLOTS ? (int64_t)G : (int64_t)S * G;
        c0 = SLOTS ? (int64_t)lane : (int64_t)sp * G + lane;
        niter = (nchunks + step - 1) / step;  // the same for every lane
    }

    // Row pointers of the tile at row0 (element by element: a copied
    // aggregate can end up in scratch memory).  Rows past n read row n-1
    // (their results are not written).
    __device__ __forceinline__ void set_rows(Rows& p, int64_t row0) const {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            int64_t r = MM ? row0 + (int64_t)rs * 4 * R + 4 * j + mi : row0 + (int64_t)rs * R + j;
            r = r < n ? r : n - 1;
            if constexpr (PAIR) r = (r >> 1) + (r & 1) * (n >> 1);
            p.c[j] = codes + r * rowbytes;
            p.s[j] = scales + r * sbytes;
        }
    }

    // Issues the loads of the lane's chunk cv (c0 + i*step in pass i).  In
    // the last pass lanes past the row end read the row's last chunk again;
    // `compute` drops that contribution.
    __device__ __forceinline__ void load(const Rows& rp, int cv, Pass& p) const {
        const int64_t c = cv < nchunks ? cv : nchunks - 1;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            load_code_chunk<CB>(rp.c[j] + c * CB, p.cw[j]);
            load_scale_bytes<FMT, CB>(rp.s[j], c, p.sb[j]);
        }
    }

    // Pointer i of a small array, by masking (a select chain over the
    // array's entries is folded back into a dynamically indexed load, which
    // puts the array in scratch memory).
    template <class T, int N>
    static __device__ __forceinline__ T* pick(T* const (&a)[N], int i) {
        uintptr_t v = 0;
#pragma unroll
        for (int k = 0; k < N; ++k) v |= reinterpret_cast<uintptr_t>(a[k]) & (uintptr_t)(-(intptr_t)(i == k));
        return reinterpret_cast<T*>(v);
    }

    // Matrix mode: the pass's R chunks through the 16 x 16 x 32 MFMA (see above).
    __device__ __forceinline__ void compute_mm(const Pass& p, int cv, const uint16_t* const (&xs)[B],
                                               const uint8_t* xlds, float (&acc)[R][NA]) const {
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x8_mm_t __attribute__((ext_vector_type(8)));
        constexpr int KSTEPS = CS::NP / 4;  // MFMA k steps (8 elements) per chunk
        const bool valid = cv < nchunks;
        const int64_t c = valid ? cv : nchunks - 1;
        // B operand: activation vector mi at this lane's chunk (zero past the batch or the row)
        uint32_t xw[CS::NP];
#pragma unroll
        for (int t = 0; t < CS::NP; ++t) xw[t] = 0u;
        if (mi < B && valid) {
            const int64_t vc = c * B + mi;
            const u32x4_t* xp = XL ? reinterpret_cast<const u32x4_t*>(xlds) + vc * CS::XQ
                                   : reinterpret_cast<const u32x4_t*>(pick(xs, mi)) + c * CS::XQ;
            const int swz = XL ? x_swizzle<FMT, CB>(vc) : 0;
#pragma unroll
            for (int q = 0; q < CS::XQ; ++q) {
                const u32x4_t v = xp[q ^ swz];
                xw[4 * q + 0] = v[0]; xw[4 * q + 1] = v[1]; xw[4 * q + 2] = v[2]; xw[4 * q + 3] = v[3];
            }
        }
        bf16x8_mm_t bx[KSTEPS];
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
            bx[t] = __builtin_bit_cast(bf16x8_mm_t, u32x4_t{xw[4 * t], xw[4 * t + 1], xw[4 * t + 2], xw[4 * t + 3]});
        bool lifted = false;
        if constexpr (FMT == kMXFP8) {
            bool lo = false;
#pragma unroll
            for (int j = 0; j < R; ++j) lo = lo || mx_lifted<FMT>(p.sb[j][0]);
            lifted = __ballot(lo) != 0;
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            // A operand: the decoded chunk of row j (zero past the row end, where
            // the re-read chunk is not this lane's to add)
            uint32_t wp[CS::NP];
            bool lo = false;
            if constexpr (FMT == kNVFP4) {
                float sc[CS::NSG];
                scale_values<FMT, CB>(p.sb[j], sc);
#pragma unroll
                for (int d = 0; d < CS::DW; ++d) {
                    const float sv = sc[(4 * d) / CS::PPS];
                    wp[4 * d + 0] = scaled_fp4x2_to_bf16x2<0>(p.cw[j][d], sv);
                    wp[4 * d + 1] = scaled_fp4x2_to_bf16x2<1>(p.cw[j][d], sv);
                    wp[4 * d + 2] = scaled_fp4x2_to_bf16x2<2>(p.cw[j][d], sv);
                    wp[4 * d + 3] = scaled_fp4x2_to_bf16x2<3>(p.cw[j][d], sv);
                }
            } else {
                const uint32_t u = p.sb[j][0];
                lo = mx_lifted<FMT>(u);
                decode_dwords_scaled<FMT, CS::DW>(p.cw[j], e8m0_exponent(lo ? u + kMx8Lift : u), wp);
            }
#pragma unroll
            for (int t = 0; t < CS::NP; ++t) wp[t] = valid ? wp[t] : 0u;
            f32x4_t d = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
            if (!lifted) {
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t)
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_mm_t, u32x4_t{wp[4 * t], wp[4 * t + 1], wp[4 * t + 2], wp[4 * t + 3]}),
                        bx[t], d, 0, 0, 0);
            } else {
                // lifted MXFP8 rows (decoded 2^3 larger) go into a sum scaled back in fp32
                f32x4_t e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    const u32x4_t w4 = {wp[4 * t], wp[4 * t + 1], wp[4 * t + 2], wp[4 * t + 3]};
                    const u32x4_t z4 = {0u, 0u, 0u, 0u};
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_mm_t, lo ? z4 : w4), bx[t], d, 0, 0, 0);
                    e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_mm_t, lo ? w4 : z4), bx[t], e, 0, 0, 0);
                }
                d += e * kMx8Unlift;
            }
            acc[j][0] = d[0]; acc[j][1] = d[1]; acc[j][2] = d[2]; acc[j][3] = d[3];
        }
    }

    // Arithmetic of the pass with chunk cv on its loaded chunks.
    __device__ __forceinline__ void compute(const Pass& p, int cv, const uint16_t* const (&xs)[B],
                                            const uint8_t* xlds, float (&acc)[R][NA]) const {
        if constexpr (MM) {
            compute_mm(p, cv, xs, xlds, acc);
            return;
        }
        const bool valid = cv < nchunks;
        const int64_t c = valid ? cv : nchunks - 1;
        uint32_t xw[B][CS::NP];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int64_t vc = (SLOTS ? (int64_t)sp : (int64_t)b) * nchunks + c;  // chunk of the staged block
            const u32x4_t* xp = XL ? reinterpret_cast<const u32x4_t*>(xlds) + vc * CS::XQ
                                   : reinterpret_cast<const u32x4_t*>(xs[b]) + c * CS::XQ;
            const int swz = XL ? x_swizzle<FMT, CB>(vc) : 0;
#pragma unroll
            for (int q = 0; q < CS::XQ; ++q) {
                const u32x4_t v = xp[q ^ swz];
                xw[b][4 * q + 0] = v[0]; xw[b][4 * q + 1] = v[1]; xw[b][4 * q + 2] = v[2]; xw[b][4 * q + 3] = v[3];
            }
        }
        // MXFP8 passes holding a block with an E8M0 byte below kMx8Lift take
        // the lifted form (a branch taken by the whole wave or by none of it)
        bool lifted = false;
        if constexpr (FMT == kMXFP8) {
            bool lo = false;
#pragma unroll
            for (int j = 0; j < R; ++j) lo = lo || mx_lifted<FMT>(p.sb[j][0]);
            lifted = __ballot(lo) != 0;
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            uint32_t wp[CS::NP];
            if constexpr (FMT == kNVFP4) {
                float sc[CS::NSG];
                scale_values<FMT, CB>(p.sb[j], sc);
                decode_dwords<FMT, CS::DW>(p.cw[j], wp);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float a = acc[j][b];
#pragma unroll
                    for (int q = 0; q < CS::NSG; ++q) {
                        float part = 0.0f;
#pragma unroll
                        for (int t = 0; t < CS::PPS; ++t) part = dot2_bf16(wp[q * CS::PPS + t], xw[b][q * CS::PPS + t], part);
                        a = __builtin_fmaf(part, sc[q], a);
                    }
                    acc[j][b] = valid ? a : acc[j][b];
                }
            } else if (!lifted) {
                decode_dwords_scaled<FMT, CS::DW>(p.cw[j], e8m0_exponent(p.sb[j][0]), wp);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float a = acc[j][b];
#pragma unroll
                    for (int t = 0; t < CS::NP; ++t) a = dot2_bf16(wp[t], xw[b][t], a);
                    acc[j][b] = valid ? a : acc[j][b];
                }
            } else {
                // a lifted MXFP8 chunk: decoded 2^3 larger, its partial sum scaled back in fp32
                const uint32_t u = p.sb[j][0];
                const bool lo = mx_lifted<FMT>(u);
                decode_dwords_scaled<FMT, CS::DW>(p.cw[j], e8m0_exponent(lo ? u + kMx8Lift : u), wp);
                const float mul = lo ? kMx8Unlift : 1.0f;
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float part = 0.0f;
#pragma unroll
                    for (int t = 0; t < CS::NP; ++t) part = dot2_bf16(wp[t], xw[b][t], part);
                    const float a = __builtin_fmaf(part, mul, acc[j][b]);
                    acc[j][b] = valid ? a : acc[j][b];
                }
            }
        }
    }

    // Sum over the G lanes and the S groups of the tile at row0 and store
    // ys[b][row] = gmul * sum (rows >= n are not written; ys[b] == nullptr
    // skips entry b).  With SLOTS the groups' sums are weighted by smul[s] and
    // groups s >= nslot are left out.
    __device__ __forceinline__ void finish(int64_t row0, float (&acc)[R][NA], float* const (&ys)[B], float gmul,
                                           float* red, const float* smul = nullptr, int nslot = S) const {
        if constexpr (MM) {
            finish_mm(row0, acc, ys, gmul, red);
            return;
        }
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[j][b] = group_sum<G>(acc[j][b]);

        if constexpr (PAIR) {
            if (lane == 0) {
                const int64_t half = n >> 1;
#pragma unroll
                for (int j = 0; j < R; j += 2) {
                    const int64_t i = (row0 + (int64_t)rs * R + j) >> 1;
                    if (i < half) {
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            if (ys[b]) {
                                const float g = acc[j][b] * gmul, u = acc[j + 1][b] * gmul;
                                ys[b][i] = g;
                                ys[b][i + half] = u;
                                act0[(ys[b] - y0) / 2 + i] = swiglu_bf16(g, u);
                            }
                        }
                    }
                }
            }
        } else if constexpr (S == 1) {
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const int64_t r = row0 + (int64_t)rs * R + j;
                    if (r < n) {
#pragma unroll
                        for (int b = 0; b < B; ++b)
                            if (ys[b]) ys[b][r] = SLOTS ? acc[j][b] * smul[0] : acc[j][b] * gmul;
                    }
                }
            }
        } else {
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int b = 0; b < B; ++b) red[((sp * T::ROWSETS + rs) * R + j) * B + b] = acc[j][b];
            }
            lds_barrier();
            for (int t = threadIdx.x; t < T::ROWSETS * R; t += kThreads) {
                const int j = t % R, set = t / R;
                const int64_t r = row0 + (int64_t)set * R + j;
                if (r < n) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        if constexpr (SLOTS) {
                            float v = red[(set * R + j) * B + b] * smul[0];
#pragma unroll
                            for (int s = 1; s < S; ++s)
                                if (s < nslot) v += red[((s * T::ROWSETS + set) * R + j) * B + b] * smul[s];
                            if (ys[b]) ys[b][r] = v;
                        } else {
                            float v = red[(set * R + j) * B + b];
#pragma unroll
                            for (int s = 1; s < S; ++s) v += red[((s * T::ROWSETS + set) * R + j) * B + b];
                            if (ys[b]) ys[b][r] = v * gmul;
                        }
                    }
                }
            }
            lds_barrier();  // `red` is rewritten by the next tile
        }
    }

    // Matrix mode: lane l holds the product rows 4q + e (q = l / 16, e = 0..3)
    // of column l % 16 for each of its R groups; the diagonal entry e = l % 4
    // is row q's sum over segment l % 4 for activation vector (l / 4) % 4.  A
    // quad reduction adds the 4 segments (fixed order), then the S waves of a
    // row group are added through LDS.
    __device__ __forceinline__ void finish_mm(int64_t row0, float (&acc)[R][NA], float* const (&ys)[B], float gmul,
                                              float* red) const {
        const int l = threadIdx.x & 63;
        const int e = l & 3, q = l >> 4;
        float v[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            // the lane's diagonal entry (register e), by selects
            float t = (e == 0 ? acc[j][0] : 0.0f) + (e == 1 ? acc[j][1] : 0.0f);
            t += (e == 2 ? acc[j][2] : 0.0f) + (e == 3 ? acc[j][3] : 0.0f);
            t += dpp_f32<kDppQuadXor1>(t);
            t += dpp_f32<kDppQuadXor2>(t);
            v[j] = t;
        }
        const bool head = e == 0;  // lane (q, vector mi) holds row q's total
        if constexpr (S == 1) {
            float* yp = pick(ys, mi);
            if (head && mi < B && yp) {
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const int64_t r = row0 + (int64_t)rs * 4 * R + 4 * j + q;
                    if (r < n) yp[r] = v[j] * gmul;
                }
            }
        } else {
            if (head) {
#pragma unroll
                for (int j = 0; j < R; ++j) red[((sp * WSETS + rs) * 4 * R + 4 * j + q) * 4 + mi] = v[j];
            }
            lds_barrier();
            for (int t = threadIdx.x; t < WSETS * 4 * R * 4; t += kThreads) {
                const int vv = t & 3, row = t >> 2;  // row within the tile: group * 4R + 4j + q
                const int64_t r = row0 + row;
                float* yp = pick(ys, vv);
                if (r < n && vv < B && yp) {
                    float sum = red[row * 4 + vv];
#pragma unroll
                    for (int s2 = 1; s2 < S; ++s2) sum += red[(s2 * WSETS * 4 * R + row) * 4 + vv];
                    yp[r] = sum * gmul;
                }
            }
            lds_barrier();  // `red` is rewritten by the next tile
        }
    }

    __device__ __forceinline__ Cursor cursor(int64_t first, int64_t row_step, int64_t count, const uint16_t* x0) const {
        Cursor u;
        u.first = first;
        u.row_step = row_step;
        u.count = count;
        u.tl = 0;
        u.il = 0;
        u.cl = (int)c0;
        set_rows(u.rl, first);
        u.dummy = reinterpret_cast<const uint8_t*>(x0);
        return u;
    }

    __device__ __forceinline__ void advance(Cursor& u) const {
        u.cl += (int)step;
        if (++u.il == niter) {
            u.il = 0;
            u.cl = (int)c0;
            ++u.tl;
            // every slot is assigned on every path (selects, not branches):
            // a store merged across branches would put the pointers in scratch
            const bool more = u.tl < u.count;
            set_rows(u.rl, u.first + (more ? u.tl : 0) * u.row_step);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                u.rl.c[j] = more ? u.rl.c[j] : u.dummy;
                u.rl.s[j] = more ? u.rl.s[j] : u.dummy;
            }
        }
    }

    // Issues the loads of passes 0 .. D-1 into ring buffers 0 .. D-1.
    template <int D>
    __device__ __forceinline__ void prime(Cursor& u, PassRing<Pass, D + 1>& ring) const {
        static_for<0, D>([&](auto d) {
            load(u.rl, u.cl, ring.template at<decltype(d)::value>());
            advance(u);
        });
    }

    // Streams the cursor's tiles as one sequence of passes, D passes ahead:
    // the loads of pass p + D are issued before the arithmetic of pass p,
    // across tile boundaries.  ring[0 .. D-1] must hold passes 0 .. D-1
    // (prime).  The ring is indexed statically (groups of D+1 passes, no
    // register copies) and no load sits inside a branch, so the compiler's
    // wait counts stay exact and D passes stay in flight.  With XL the
    // activations must already be in `xlds` (stage_x); `red` is LDS scratch
    // of S*ROWSETS*R*B floats (unused when S == 1).
    template <int D>
    __device__ __forceinline__ void run(Cursor& u, PassRing<Pass, D + 1>& ring, const uint16_t* const (&xs)[B],
                                        float* const (&ys)[B], float gmul, float* red, const uint8_t* xlds,
                                        const float* smul = nullptr, int nslot = S) const {
        const int64_t total = u.count * niter;
        // compute cursor: tile tc, pass ic, chunk cc
        int64_t tc = 0, ic = 0;
        int cc = (int)c0;
        float acc[R][NA];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < NA; ++b) acc[j][b] = 0.0f;
        auto arith = [&](const Pass& cur) {
            compute(cur, cc, xs, xlds, acc);
            cc += (int)step;
            if (++ic == niter) {  // tile done: reduce and store
                finish(u.first + tc * u.row_step, acc, ys, gmul, red, smul, nslot);
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int b = 0; b < NA; ++b) acc[j][b] = 0.0f;
                ic = 0;
                cc = (int)c0;
                ++tc;
            }
        };
        int64_t P = 0;
        for (; P + (D + 1) <= total; P += D + 1) {
            static_for<0, D + 1>([&](auto w) {
                constexpr int W = decltype(w)::value;
                load(u.rl, u.cl, ring.template at<(W + D) % (D + 1)>());
                advance(u);
                arith(ring.template at<W>());
            });
        }
        // the last passes are already loaded
        static_for<0, D>([&](auto w) {
            constexpr int W = decltype(w)::value;
            if (P + W < total) arith(ring.template at<W>());
        });
    }
};

}  // namespace mxq
