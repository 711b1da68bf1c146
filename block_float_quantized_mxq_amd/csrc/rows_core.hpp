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
// Per 16-byte chunk: MXFP4 = one 32-element block (one E8M0 byte), MXFP8 = half
// a 32-element block, NVFP4 = two 16-element blocks (two E4M3 bytes).  An
// 8-byte chunk is used for NVFP4 rows whose byte length is not a multiple of 16.
// The block scale multiplies the block's fp32 partial sum; NVFP4's per-tensor
// scale multiplies the final sum.
//
// Activations: each lane needs the activation chunk matching its code chunk
// for every batch entry.  With XL the workgroup first copies x[B][k] into LDS
// (one padded 16-byte slot after every chunk, so the 16 lanes of a group hit
// distinct banks) and the loop reads it from there; otherwise the loop loads
// it from global memory (L1/L2 resident), once per chunk for all R rows.
#pragma once

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
    static constexpr int XQ = KPC * 2 / 16;                        // 16-byte activation loads per chunk
    static constexpr int XSTRIDE = XQ * 16 + 16;                   // LDS bytes per staged activation chunk
};

// LDS layout of staged activations: per batch entry, chunks in groups of XG
// (XG = 1 for the row-tile kernels), each group
// followed by 16 bytes of padding, so that lanes reading the same slot of
// different groups fall on distinct banks.
template <int FMT, int CB, int XG>
__host__ __device__ constexpr int64_t x_group_bytes() {
    return (int64_t)XG * ChunkShape<FMT, CB>::XQ * 16 + 16;
}
template <int FMT, int CB, int XG>
__host__ __device__ constexpr int64_t x_lds_offset(int64_t c) {
    return (c / XG) * x_group_bytes<FMT, CB, XG>() + (c % XG) * ChunkShape<FMT, CB>::XQ * 16;
}
template <int FMT, int CB, int XG>
__host__ __device__ constexpr int64_t x_batch_bytes(int64_t k) {
    return ((code_bytes_per_row(FMT, k) / CB + XG - 1) / XG) * x_group_bytes<FMT, CB, XG>();
}

// LDS bytes needed to stage x[B][k].
template <int FMT, int CB, int XG = 1>
__host__ __device__ constexpr int64_t x_lds_bytes(int64_t k, int b) {
    return (int64_t)b * x_batch_bytes<FMT, CB, XG>(k);
}

// Weights are read exactly once per call: load them with the nontemporal hint
// so they do not displace the activations from the caches.
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

__device__ __forceinline__ uint32_t load_scale_byte(const uint8_t* p) { return __builtin_nontemporal_load(p); }

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

// Copies x[B][k] into LDS (layout above).  Every thread of the workgroup must
// call it; it ends with a barrier.
template <int FMT, int CB, int B, int XG = 1>
__device__ __forceinline__ void stage_x(const uint16_t* const (&xs)[B], int64_t k, uint8_t* xlds) {
    using CS = ChunkShape<FMT, CB>;
    const int64_t nchunks = code_bytes_per_row(FMT, k) / CB;
    const int64_t pieces = nchunks * CS::XQ;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(xs[b]);
        uint8_t* dst = xlds + (int64_t)b * x_batch_bytes<FMT, CB, XG>(k);
        for (int64_t t = threadIdx.x; t < pieces; t += kThreads) {
            const int64_t c = t / CS::XQ, q = t % CS::XQ;
            *reinterpret_cast<u32x4_t*>(dst + x_lds_offset<FMT, CB, XG>(c) + 16 * q) = src[t];
        }
    }
    __syncthreads();
}

// Computes ys[b][row] = gmul * sum_k W[row][k] * xs[b][k] for the ROWS rows
// starting at row0 (rows >= n are neither read nor written; ys[b] == nullptr
// skips batch entry b).  Every thread of the workgroup must call it.  `red`
// is LDS scratch of S*ROWSETS*R*B floats (unused when S == 1); with XL the
// activations must already be staged in `xlds` (stage_x).  The function may be
// called repeatedly (one row tile after another) by the same workgroup.
template <int FMT, int CB, int B, int G, int S, int R, bool XL>
__device__ __forceinline__ void rows_core(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                          int64_t n, int64_t k, int64_t row0, const uint16_t* const (&xs)[B],
                                          float* const (&ys)[B], float gmul, float* red, uint8_t* xlds) {
    using CS = ChunkShape<FMT, CB>;
    using T = RowTile<G, S, R>;
    const int tid = threadIdx.x;
    const int lane = tid % G, gid = tid / G, rs = gid / S, sp = gid % S;
    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t sbytes = k / CS::BS;
    const int64_t nchunks = rowbytes / CB;

    const uint8_t* crow[R];
    const uint8_t* srow[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        int64_t r = row0 + (int64_t)rs * R + j;
        r = r < n ? r : n - 1;
        crow[j] = codes + r * rowbytes;
        srow[j] = scales + r * sbytes;
    }
    float acc[R][B];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[j][b] = 0.0f;

#pragma unroll 2
    for (int64_t c = (int64_t)sp * G + lane; c < nchunks; c += (int64_t)S * G) {
        uint32_t cw[R][CS::DW];
        float sc[R][CS::NSG];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            load_code_chunk<CB>(crow[j] + c * CB, cw[j]);
            load_chunk_scales<FMT, CB>(srow[j], c, sc[j]);
        }
        uint32_t xw[B][CS::NP];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint8_t* xp = XL ? xlds + (int64_t)b * nchunks * CS::XSTRIDE + x_lds_offset<FMT, CB, 1>(c)
                                   : reinterpret_cast<const uint8_t*>(xs[b]) + c * (CS::KPC * 2);
#pragma unroll
            for (int q = 0; q < CS::XQ; ++q) {
                u32x4_t v = *reinterpret_cast<const u32x4_t*>(xp + 16 * q);
                xw[b][4 * q + 0] = v[0]; xw[b][4 * q + 1] = v[1]; xw[b][4 * q + 2] = v[2]; xw[b][4 * q + 3] = v[3];
            }
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            uint32_t wp[CS::NP];
            decode_dwords<FMT, CS::DW>(cw[j], wp);
#pragma unroll
            for (int b = 0; b < B; ++b) {
#pragma unroll
                for (int q = 0; q < CS::NSG; ++q) {
                    float part = 0.0f;
#pragma unroll
                    for (int t = 0; t < CS::PPS; ++t) part = dot2_bf16(wp[q * CS::PPS + t], xw[b][q * CS::PPS + t], part);
                    acc[j][b] = __builtin_fmaf(part, sc[j][q], acc[j][b]);
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[j][b] = group_sum<G>(acc[j][b]);

    if constexpr (S == 1) {
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int64_t r = row0 + (int64_t)rs * R + j;
                if (r < n) {
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        if (ys[b]) ys[b][r] = acc[j][b] * gmul;
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
        __syncthreads();
        for (int t = tid; t < T::ROWSETS * R; t += kThreads) {
            const int j = t % R, set = t / R;
            const int64_t r = row0 + (int64_t)set * R + j;
            if (r < n) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float v = red[(set * R + j) * B + b];
#pragma unroll
                    for (int s = 1; s < S; ++s) v += red[((s * T::ROWSETS + set) * R + j) * B + b];
                    if (ys[b]) ys[b][r] = v * gmul;
                }
            }
        }
        __syncthreads();  // `red` is rewritten by the next tile
    }
}

}  // namespace mxq
