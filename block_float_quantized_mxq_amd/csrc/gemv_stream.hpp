// gemv_stream.hpp -- the dense GEMV kernel: a software-pipelined weight stream.
//
// y[b][i] = sum_k W[i][k] * x[b][k] reads every weight byte once, so it is
// bound by HBM bandwidth ("The memory wall" section of the "MLxcel 0.8
// release" post: the decode ceiling is bandwidth / weight bytes).  On MI355X
// the read ceiling is only reached with a few tens of KB of reads in flight
// per CU, so the kernel is organised around keeping loads outstanding:
//
//  * Each group of G lanes (64: one wave; 16 or 32 for short rows) streams
//    blocks of P adjacent rows as one contiguous run of 16-byte chunks, blocks
//    dealt round-robin over the grid's groups; every load instruction of a
//    group reads G*16 contiguous bytes.
//  * The (row, chunk) items of a lane form one stream.  A ring of D registers
//    keeps the next D items' code loads in flight (nontemporal hint: the
//    weights are read once); loads are unconditional (items past the end or
//    past the row are clamped to a valid address and masked with a zero
//    scale), so the compiler can count outstanding loads exactly.
//  * When a lane consumes the last item of a block, the group sums its G
//    partials of each row (DPP row operations, plus lane shuffles beyond 16)
//    and lane 0 writes y.  No LDS reduction
//    and no barrier sit inside the stream.
//  * Activations: with XL the workgroup copies x[B][k] into LDS once (a padded
//    slot per chunk keeps the 16 lanes on distinct banks); otherwise each lane
//    loads its activation chunk from global memory (L2 resident).
//
// Decode and contraction per chunk are the same as in rows_core.hpp: the
// E2M1 / E4M3 codes become exact bf16 pairs, v_dot2 accumulates a block
// partial in fp32, and the block scale multiplies that partial (one fma).
#pragma once

#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {


// Contraction of one decoded chunk with the B activation chunks at chunk
// index cc, accumulated into acc with the chunk's scale multipliers.
template <int FMT, int CB, int B, bool XL>
__device__ __forceinline__ void stream_consume(const uint32_t (&cw)[ChunkShape<FMT, CB>::DW],
                                               const float (&sc)[ChunkShape<FMT, CB>::NSG], int64_t cc,
                                               int64_t nchunks, const uint8_t* xlds,
                                               const uint16_t* const (&xs)[B], float (&acc)[B]) {
    using CS = ChunkShape<FMT, CB>;
    uint32_t wp[CS::NP];
    decode_dwords<FMT, CS::DW>(cw, wp);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        uint32_t xw[CS::NP];
        const uint8_t* xp = XL ? xlds + ((int64_t)b * nchunks + cc) * CS::XSTRIDE
                               : reinterpret_cast<const uint8_t*>(xs[b]) + cc * (CS::KPC * 2);
#pragma unroll
        for (int q = 0; q < CS::XQ; ++q) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xp + 16 * q);
            xw[4 * q + 0] = v[0]; xw[4 * q + 1] = v[1]; xw[4 * q + 2] = v[2]; xw[4 * q + 3] = v[3];
        }
#pragma unroll
        for (int q = 0; q < CS::NSG; ++q) {
            float part = 0.0f;
#pragma unroll
            for (int t = 0; t < CS::PPS; ++t) part = dot2_bf16(wp[q * CS::PPS + t], xw[q * CS::PPS + t], part);
            acc[b] = __builtin_fmaf(part, sc[q], acc[b]);
        }
    }
}

// Scale-byte offset of chunk c counted from the start of the scale rows (the
// scale layout makes it a function of the global chunk index).
template <int FMT, int CB>
__device__ __forceinline__ int64_t scale_offset(int64_t c) {
    if constexpr (FMT == kMXFP8) return c >> 1;
    else if constexpr (FMT == kNVFP4 && CB == 16) return 2 * c;
    else return c;
}

template <int FMT, int CB>
__device__ __forceinline__ void load_scale_at(const uint8_t* sp, uint32_t (&sb)[ChunkShape<FMT, CB>::NSG]) {
    sb[0] = load_scale_byte(sp);
    if constexpr (ChunkShape<FMT, CB>::NSG == 2) sb[1] = load_scale_byte(sp + 1);
}

// Work unit: a block of P adjacent rows, read as one contiguous run of
// P * nchunks 16-byte chunks by a group of G lanes (P * nchunks must be a
// multiple of G, and G <= nchunks): lane l takes chunks l, l+G, l+2G, ... of
// the block, so every load instruction of the group covers G*16 contiguous
// bytes and consecutive items of a lane sit at a fixed stride.  Blocks are
// dealt round-robin over the grid's GT groups (block g, g+GT, ...), so at any
// moment the GPU reads a window of about GT consecutive blocks and sweeps the
// matrix front to back, which keeps DRAM accesses local.  A lane tracks which
// row of the block its chunk belongs to and keeps one accumulator per row.
template <int FMT, int CB, int B, int G, int P, int D, bool XL>
__global__ __launch_bounds__(kThreads) void gemv_stream_kernel(const uint8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               const float* __restrict__ gscale,
                                                               const uint16_t* __restrict__ x,
                                                               float* __restrict__ y, int64_t n, int64_t k,
                                                               int batch) {
    using CS = ChunkShape<FMT, CB>;
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
    const int tid = threadIdx.x;
    const int lane = tid % G;
    const int64_t group = (int64_t)blockIdx.x * (kThreads / G) + tid / G;
    const int64_t gt = (int64_t)gridDim.x * (kThreads / G);

    const uint16_t* xs[B];
    float* ys[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        xs[b] = x + (int64_t)(b < batch ? b : 0) * k;
        ys[b] = b < batch ? y + (int64_t)b * n : nullptr;
    }

    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const int64_t nchunks = rowbytes / CB;
    const int64_t ipb = P * nchunks / G;              // items per block per lane
    const int64_t nblocks = (n + P - 1) / P;
    const int64_t myblocks = group < nblocks ? (nblocks - group + gt - 1) / gt : 0;
    const int64_t total = myblocks * ipb;
    const float gmul = (FMT == kNVFP4) ? gscale[0] : 1.0f;
    const int64_t nchunks_all = n * nchunks;          // chunks in the whole matrix

    uint32_t ring[D][CS::DW];
    uint32_t sring[D][CS::NSG];

    // Load state: global chunk index of the lane's next item; past the end of
    // the matrix it is clamped to the last chunk (valid memory, never used).
    int64_t lblock = group < nblocks ? group : nblocks - 1;
    int64_t lchunk = lblock * P * nchunks + lane;     // global chunk index
    int64_t lt = 0;                                   // item within block
    const int64_t bstep = (gt - 1) * P * nchunks + G; // from a block's last item to the next block's first
    auto load_item = [&](int d) {
        const int64_t c = lchunk < nchunks_all ? lchunk : nchunks_all - 1;
        load_code_chunk<CB>(codes + c * CB, ring[d]);
        load_scale_at<FMT, CB>(scales + scale_offset<FMT, CB>(c), sring[d]);
        if (++lt == ipb) {
            lt = 0;
            lchunk += bstep;
        } else {
            lchunk += G;
        }
    };

    // The first D loads go out before the activations are staged, so the
    // staging latency overlaps the weight fetch.
#pragma unroll
    for (int d = 0; d < D; ++d) load_item(d);
    if constexpr (XL) stage_x<FMT, CB, B>(xs, k, xlds);

    float acc[P][B];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[p][b] = 0.0f;
    // Consume state: block, item within block, row within block and chunk
    // within row of the lane's current item.
    int64_t cblock = group, ct = 0, cir = lane;
    int crib = 0;

    for (int64_t i = 0; i < total; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float sc[CS::NSG];
            scale_values<FMT, CB>(sring[d], sc);
            if constexpr (P == 1) {
                stream_consume<FMT, CB, B, XL>(ring[d], sc, cir, nchunks, xlds, xs, acc[0]);
            } else {
                float part[B];
#pragma unroll
                for (int b = 0; b < B; ++b) part[b] = 0.0f;
                stream_consume<FMT, CB, B, XL>(ring[d], sc, cir, nchunks, xlds, xs, part);
#pragma unroll
                for (int p = 0; p < P; ++p)
#pragma unroll
                    for (int b = 0; b < B; ++b) acc[p][b] += (crib == p) ? part[b] : 0.0f;
            }
            if (++ct == ipb) {  // block complete: same for all G lanes of the group
                const int64_t row0 = cblock * P;
#pragma unroll
                for (int p = 0; p < P; ++p)
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float sum = group_sum<G>(acc[p][b]);
                        if (lane == 0 && row0 + p < n && ys[b]) ys[b][row0 + p] = sum * gmul;
                        acc[p][b] = 0.0f;
                    }
                ct = 0;
                cblock += gt;
                cir = lane;
                crib = 0;
            } else {
                cir += G;
                if (cir >= nchunks) {
                    cir -= nchunks;
                    ++crib;
                }
            }
            load_item(d);  // refill the slot with the item D ahead
        }
    }
}

}  // namespace mxq
