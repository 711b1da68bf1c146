// moe_impl.hpp -- expert-indexed MoE GEMV: the kernel and its launcher for
// one format; each format is instantiated in its own translation unit
// (moe_<format>.hip) so the instances compile in parallel.
//
// Each (token, slot) pair routed to expert e needs W[e] . x_ts.  The section
// "Unified memory" of the "MLxcel 0.8 release" post (and slide 4 of the talk)
// gives the property this kernel is built on: a token reads only its active
// experts.  Here every routed expert's rows are streamed exactly once per call,
// however many pairs route to it: the grid is (row tile, routing position p);
// the workgroup at position p returns at once if an earlier position holds the
// same expert, and otherwise gathers every later position with that expert
// and runs them as one batch through the shared streaming loop.  Dedupe and
// gather happen in-kernel, so there is no host synchronisation and no
// scratch memory.  A position whose id is outside [0, E) gets NaN outputs.
#pragma once

#include "kernels.hpp"
#include "moe_route.hpp"
#include "rows_core.hpp"

namespace mxq {

// Routing positions per call (MXQ_MAX_BATCH * MXQ_MAX_TOPK): two ids per lane.
constexpr int kMaxPairs = 8 * 16;
static_assert(kMaxPairs <= 128, "the kernel holds two routing ids per lane");
constexpr int64_t kMoeMaxXLds = 64 * 1024;

// Passes each lane keeps in flight ahead of its arithmetic (measured on
// MI355X: more than one does not help even at one token).
#ifndef MXQ_MOE_AHEAD
#define MXQ_MOE_AHEAD 1
#endif
constexpr int kMoeAhead = MXQ_MOE_AHEAD;

// Pairs per round: 1 at one token, else 2.  A token's experts are distinct, so
// an expert gets at most `tokens` pairs, and with 128 experts rarely more than
// one or two; an expert with more pairs than the cap takes extra rounds (its
// rows come from L2 the second time).  The small cap keeps the registers of a
// two-vector loop (MI355X, 30B-A3B bank, against rounds of min(8, tokens)
// rounded up to a power of two: 4 tokens gate/up 15.9 -> 13.7 us, down 12.3 ->
// 9.5 us; 8 tokens 36.7 -> 23.4 us, 22.9 -> 16.1 us; rounds of one pair were
// within 5% at 2 and 4 tokens).  LDS holds one round's activations.
static int moe_round_cap(int64_t tokens) {
    return tokens <= 1 ? 1 : 2;
}

// Takes the next routing position from the two 64-bit masks (positions 0..63
// in m0, 64..127 in m1), lowest first; -1 when both are empty.
__device__ __forceinline__ int next_position(uint64_t& m0, uint64_t& m1) {
    if (m0) {
        const int q = __builtin_ctzll(m0);
        m0 &= m0 - 1;
        return q;
    }
    if (m1) {
        const int q = 64 + __builtin_ctzll(m1);
        m1 &= m1 - 1;
        return q;
    }
    return -1;
}

// One round: the B positions in q[0..B) (q < 0: unused slot) contracted with
// the expert's row tile, with activations staged in LDS when XL.  The ring
// holds the tile's first passes on entry.
template <int FMT, int CB, int B, int G, int S, int R, bool XL, bool PAIR, int D>
__device__ __forceinline__ void moe_round(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                          int64_t row0, const int (&q)[8], const uint16_t* x, int x_per_slot,
                                          int64_t topk, float* y, uint16_t* act, float gmul, float* red,
                                          uint8_t* xlds, RowCursor<R>& cur,
                                          PassRing<RowPass<FMT, CB, R>, D + 1>& ring) {
    const uint16_t* xs[B];
    float* ys[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int qq = q[b] >= 0 ? q[b] : q[0];
        const int64_t xrow = x_per_slot ? (int64_t)qq : (int64_t)qq / topk;
        xs[b] = x + xrow * k;
        ys[b] = q[b] >= 0 ? y + (int64_t)q[b] * n : nullptr;
    }
    if constexpr (XL) stage_x<FMT, CB, B>(xs, k, xlds);
    RowEngine<FMT, CB, B, G, S, R, XL, false, false, PAIR> eng(codes, scales, n, k);
    eng.y0 = y;
    eng.act0 = act;
    eng.template run<D>(cur, ring, xs, ys, gmul, red, xlds);
}

// Row tiles through the streaming engine; grid (row tile, routing position p).
// Every wave reads the routing ids itself (two per lane) and finds, with
// ballots, whether an earlier position holds the same expert and which later
// positions share it: no LDS and no barrier before the weight loads start.
// PAIR: the rows are a SwiGLU layer's gate rows then up rows, and position q
// also gets its activations bf16(silu(gate) * up) at act + q n/2 (a position
// with an invalid id gets NaN outputs and no activations).
// RNS > 0: the kernel routes in place (moe_route.hpp, RNS logits per lane):
// wave w of every workgroup routes tokens w, w + 4, ... into LDS, and
// workgroup (0, 0) also writes the ids and weights to ids_out / weights_out.
// Every workgroup computes the same routing, so they all agree on it; this
// spares the routing launch.
// At least 3 waves per SIMD: the two-vector loops sit just under the 170
// registers that allow 3 (a few more registers would halve the waves in
// flight: MI355X, 30B-A3B gate/up with SwiGLU, 2 tokens 8 -> 12 us).
template <int FMT, int CB, int G, int S, int R, bool XL, int RC, bool PAIR, int RNS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void moe_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ gscale,
                                                       const int32_t* __restrict__ ids,
                                                       const uint16_t* __restrict__ x, int x_per_slot,
                                                       float* __restrict__ y, uint16_t* __restrict__ act,
                                                       int64_t experts, int64_t n, int64_t k, int pairs,
                                                       int64_t topk, const float* __restrict__ logits, int renorm,
                                                       int32_t* __restrict__ ids_out, float* __restrict__ weights_out) {
    using T = RowTile<G, S, R>;
    __shared__ float red[S > 1 ? S * T::ROWSETS * R * 8 : 1];
    __shared__ int32_t rids[RNS > 0 ? kMaxPairs : 1];
    __shared__ float rwts[RNS > 0 ? kMaxPairs : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
    const int p = blockIdx.y;
    const int64_t row0 = (int64_t)blockIdx.x * T::ROWS;
    const int wl = threadIdx.x & 63;
    int v0, v1;
    if constexpr (RNS > 0) {
        const int tokens = pairs / (int)topk;
        for (int t = threadIdx.x >> 6; t < tokens; t += kThreads / 64)
            route_wave<RNS>(logits + (int64_t)t * experts, (int)experts, (int)topk, renorm, rids + t * topk,
                            rwts + t * topk);
        __syncthreads();
        if (blockIdx.x == 0 && blockIdx.y == 0)
            for (int i = threadIdx.x; i < pairs; i += kThreads) {
                ids_out[i] = rids[i];
                weights_out[i] = rwts[i];
            }
        v0 = wl < pairs ? rids[wl] : -1;
        v1 = wl + 64 < pairs ? rids[wl + 64] : -1;
    } else {
        v0 = wl < pairs ? ids[wl] : -1;
        v1 = wl + 64 < pairs ? ids[wl + 64] : -1;
    }
    const int e = __shfl(p < 64 ? v0 : v1, p & 63, 64);
    if (e < 0 || (int64_t)e >= experts) {
        for (int t = threadIdx.x; t < T::ROWS; t += kThreads)
            if (row0 + t < n) y[(int64_t)p * n + row0 + t] = __builtin_nanf("");
        return;
    }
    const uint64_t below0 = p >= 64 ? ~0ull : ((1ull << p) - 1ull);
    const uint64_t below1 = p >= 64 ? ((1ull << (p - 64)) - 1ull) : 0ull;
    uint64_t m0 = __ballot(v0 == e), m1 = __ballot(v1 == e);
    if ((m0 & below0) | (m1 & below1)) return;  // an earlier position streams this expert
    m0 &= ~below0;
    m1 &= ~below1;
    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const uint8_t* ecodes = codes + (int64_t)e * n * rowbytes;
    const uint8_t* escales = scales + (int64_t)e * n * (k / BlockSize<FMT>::value);
    // Weights first: the first passes are in flight while the activations load.
    using Geo = RowEngine<FMT, CB, 1, G, S, R, XL, false, false, PAIR>;
    const Geo geo(ecodes, escales, n, k);
    RowCursor<R> cur = geo.cursor(row0, 0, 1, x);
    const RowCursor<R> start = cur;
    PassRing<RowPass<FMT, CB, R>, kMoeAhead + 1> ring;
    geo.template prime<kMoeAhead>(cur, ring);
    const float gmul = (FMT == kNVFP4) ? gscale[e] : 1.0f;
    bool first = true;
    while (m0 | m1) {
        int q[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) q[b] = b < RC ? next_position(m0, m1) : -1;
        if (!first) {
            lds_barrier();  // the previous round's activations are no longer read
            cur = start;
            geo.template prime<kMoeAhead>(cur, ring);
        }
        first = false;
        // at most RC pairs per round (the LDS is sized for RC vectors); only
        // the batch sizes up to RC are compiled, so a one-token launch keeps
        // the registers of a one-vector loop
        if (RC == 1 || q[1] < 0) {
            moe_round<FMT, CB, 1, G, S, R, XL, PAIR, kMoeAhead>(ecodes, escales, n, k, row0, q, x, x_per_slot, topk, y, act, gmul, red, xlds, cur, ring);
        } else if constexpr (RC >= 2) {
            if (RC == 2 || q[2] < 0) {
                moe_round<FMT, CB, 2, G, S, R, XL, PAIR, kMoeAhead>(ecodes, escales, n, k, row0, q, x, x_per_slot, topk, y, act, gmul, red, xlds, cur, ring);
            } else if constexpr (RC >= 4) {
                if (RC == 4 || q[4] < 0)
                    moe_round<FMT, CB, 4, G, S, R, XL, PAIR, kMoeAhead>(ecodes, escales, n, k, row0, q, x, x_per_slot, topk, y, act, gmul, red, xlds, cur, ring);
                else
                    moe_round<FMT, CB, 8, G, S, R, XL, PAIR, kMoeAhead>(ecodes, escales, n, k, row0, q, x, x_per_slot, topk, y, act, gmul, red, xlds, cur, ring);
            }
        }
    }
}

template <int FMT, int CB, int G, int S, int R, int RC, bool PAIR, int RNS>
static void launch_moe_rc(const MoeArgs& a, hipStream_t st) {
    using T = RowTile<G, S, R>;
    const int64_t tiles = (a.n + T::ROWS - 1) / T::ROWS;
    const int pairs = (int)(a.tokens * a.topk);
    const int64_t lds = x_lds_bytes<FMT, CB>(a.k, RC);
    if (lds <= kMoeMaxXLds)
        hipLaunchKernelGGL((moe_kernel<FMT, CB, G, S, R, true, RC, PAIR, RNS>), dim3((unsigned)tiles, (unsigned)pairs),
                           dim3(kThreads), (size_t)lds, st, a.codes, a.scales, a.gscale, a.ids, a.x, a.x_per_slot, a.y,
                           a.act, a.experts, a.n, a.k, pairs, a.topk, a.logits, a.renorm, a.ids_out, a.weights_out);
    else
        hipLaunchKernelGGL((moe_kernel<FMT, CB, G, S, R, false, RC, PAIR, RNS>), dim3((unsigned)tiles, (unsigned)pairs),
                           dim3(kThreads), 0, st, a.codes, a.scales, a.gscale, a.ids, a.x, a.x_per_slot, a.y, a.act,
                           a.experts, a.n, a.k, pairs, a.topk, a.logits, a.renorm, a.ids_out, a.weights_out);
}

template <int FMT, int CB, int G, int S, int R, bool PAIR = false, int RNS = 0>
static void launch_moe_inst(const MoeArgs& a, hipStream_t st) {
    if (moe_round_cap(a.tokens) == 1) launch_moe_rc<FMT, CB, G, S, R, 1, PAIR, RNS>(a, st);
    else launch_moe_rc<FMT, CB, G, S, R, 2, PAIR, RNS>(a, st);
}

// The SwiGLU (paired-row) form, routing in place when a.logits is set: two
// logits per lane up to 128 experts, else 16 (1024 experts).
template <int FMT, int CB, int G>
static void launch_moe_pair(const MoeArgs& a, hipStream_t st) {
    if (!a.logits) launch_moe_inst<FMT, CB, G, 1, 2, true, 0>(a, st);
    else if (a.experts <= 128) launch_moe_inst<FMT, CB, G, 1, 2, true, 2>(a, st);
    else launch_moe_inst<FMT, CB, G, 1, 2, true, kRouteSlots>(a, st);
}

// Tile shape: lanes per row (g), k split (s), rows per lane (r), from the
// MI355X measurements: rows of >= 64 chunks take 16 lanes and 2 rows per
// lane up to four tokens and 8 lanes with one row per lane beyond; shorter
// rows take 8 lanes up to two tokens and 4 lanes beyond (more rows per
// workgroup for the same activations).
template <int FMT, int CB>
static bool launch_moe_cb(const MoeArgs& a, hipStream_t st) {
    const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
    if (a.act) {
        // SwiGLU pairs: two rows per lane, the lanes per row of the plain shapes
        if (a.n % 2) return false;
        if (a.logits && a.experts > kRouteMaxExperts) return false;
        if (nchunks >= 64 && a.tokens <= 4) launch_moe_pair<FMT, CB, 16>(a, st);
        else if (nchunks >= 8) launch_moe_pair<FMT, CB, 8>(a, st);
        else launch_moe_pair<FMT, CB, 4>(a, st);
        return true;
    }
    if (a.logits) return false;  // in-place routing only in the SwiGLU form
    int g = 16, sp = 1, r = 2;
    if (nchunks < 64) {
        r = 1;
        g = (a.tokens <= 2 && nchunks >= 8) ? 8 : 4;
    } else if (a.tokens >= 5) {
        g = 8;
        r = 1;
    }
#define MXQ_MOE_CASE(G_, S_, R_)                        \
    if (g == G_ && sp == S_ && r == R_) {              \
        launch_moe_inst<FMT, CB, G_, S_, R_>(a, st);   \
        return true;                                   \
    }
    MXQ_MOE_SHAPES(MXQ_MOE_CASE)
#undef MXQ_MOE_CASE
    return false;
}

}  // namespace mxq
