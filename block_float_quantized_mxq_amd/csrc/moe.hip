// moe.hip -- expert-indexed MoE GEMV.
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
#include <cstdio>
#include <cstdlib>

#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

constexpr int kMaxPairs = 8 * 16;  // MXQ_MAX_BATCH * MXQ_MAX_TOPK
constexpr int64_t kMoeMaxXLds = 64 * 1024;

// Pairs per round: at most one per token when a token's experts are distinct,
// so rounds of min(8, tokens) pairs (rounded up to 1, 2, 4, 8); repeated ids
// only add rounds.  LDS holds one round's activations.
static int moe_round_cap(int64_t tokens) {
    return tokens <= 1 ? 1 : (tokens <= 2 ? 2 : (tokens <= 4 ? 4 : 8));
}

// One round: up to B pairs routed to the same expert, contracted with the
// expert's row tile.  With XL their activations are first staged in LDS.
template <int FMT, int CB, int B, int G, int S, int R, bool XL>
__device__ __forceinline__ void moe_batch(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                          int64_t row0, const int* sel, int cnt, const uint16_t* x,
                                          int x_per_slot, int64_t topk, float* y, float gmul, float* red,
                                          uint8_t* xlds) {
    const uint16_t* xs[B];
    float* ys[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int q = sel[b < cnt ? b : 0];
        const int64_t xrow = x_per_slot ? (int64_t)q : (int64_t)q / topk;
        xs[b] = x + xrow * k;
        ys[b] = b < cnt ? y + (int64_t)q * n : nullptr;
    }
    if constexpr (XL) stage_x<FMT, CB, B>(xs, k, xlds);
    rows_core<FMT, CB, B, G, S, R, XL>(codes, scales, n, k, row0, xs, ys, gmul, red, xlds);
}

// Shared setup of both MoE kernels: the routing ids go to LDS in parallel;
// returns the expert of position p, or -1 when this workgroup has nothing to
// do (an earlier position holds the same expert, or the id is invalid, in
// which case the NaN rows are written here).  sel[0..nsel) lists every
// position >= p routed to the same expert.
template <int ROWS>
__device__ __forceinline__ int moe_setup(const int32_t* __restrict__ ids, int pairs, int p, int64_t experts,
                                         int64_t n, int64_t row0, float* __restrict__ y, int* sids, int* sel,
                                         int* nsel) {
    for (int t = threadIdx.x; t < pairs; t += kThreads) sids[t] = ids[t];
    __syncthreads();
    const int e = sids[p];
    if (e < 0 || (int64_t)e >= experts) {
        for (int t = threadIdx.x; t < ROWS; t += kThreads)
            if (row0 + t < n) y[(int64_t)p * n + row0 + t] = __builtin_nanf("");
        return -1;
    }
    for (int q = 0; q < p; ++q)
        if (sids[q] == e) return -1;  // an earlier position streams this expert
    if (threadIdx.x == 0) {
        int c = 0;
        for (int q = p; q < pairs; ++q)
            if (sids[q] == e) sel[c++] = q;
        *nsel = c;
    }
    __syncthreads();
    return e;
}

// Row tiles through rows_core; grid (row tile, routing position p).
template <int FMT, int CB, int G, int S, int R, bool XL>
__global__ __launch_bounds__(kThreads) void moe_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ gscale,
                                                       const int32_t* __restrict__ ids,
                                                       const uint16_t* __restrict__ x, int x_per_slot,
                                                       float* __restrict__ y, int64_t experts, int64_t n, int64_t k,
                                                       int pairs, int64_t topk, int round_cap) {
    using T = RowTile<G, S, R>;
    __shared__ int sids[kMaxPairs];
    __shared__ int sel[kMaxPairs];
    __shared__ int nsel;
    __shared__ float red[S > 1 ? S * T::ROWSETS * R * 8 : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
    const int p = blockIdx.y;
    const int64_t row0 = (int64_t)blockIdx.x * T::ROWS;
    const int e = moe_setup<T::ROWS>(ids, pairs, p, experts, n, row0, y, sids, sel, &nsel);
    if (e < 0) return;
    const int total = nsel;
    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const uint8_t* ecodes = codes + (int64_t)e * n * rowbytes;
    const uint8_t* escales = scales + (int64_t)e * n * (k / BlockSize<FMT>::value);
    const float gmul = (FMT == kNVFP4) ? gscale[e] : 1.0f;
    for (int base = 0; base < total; base += round_cap) {
        if (base > 0) __syncthreads();  // LDS of the previous round fully consumed
        const int cnt = total - base < round_cap ? total - base : round_cap;
        const int* s = sel + base;
        // the LDS of a round is sized for round_cap vectors, and cnt <= round_cap
        if (cnt == 1)
            moe_batch<FMT, CB, 1, G, S, R, XL>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul, red, xlds);
        else if (cnt == 2)
            moe_batch<FMT, CB, 2, G, S, R, XL>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul, red, xlds);
        else if (cnt <= 4)
            moe_batch<FMT, CB, 4, G, S, R, XL>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul, red, xlds);
        else
            moe_batch<FMT, CB, 8, G, S, R, XL>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul, red, xlds);
    }
}

template <int FMT, int CB, int G, int S, int R>
static void launch_moe_inst(const MoeArgs& a, hipStream_t st) {
    using T = RowTile<G, S, R>;
    const int64_t tiles = (a.n + T::ROWS - 1) / T::ROWS;
    const int pairs = (int)(a.tokens * a.topk);
    const int round_cap = moe_round_cap(a.tokens);
    const int64_t lds = x_lds_bytes<FMT, CB>(a.k, round_cap);
    if (lds <= kMoeMaxXLds)
        hipLaunchKernelGGL((moe_kernel<FMT, CB, G, S, R, true>), dim3((unsigned)tiles, (unsigned)pairs), dim3(kThreads),
                           (size_t)lds, st, a.codes, a.scales, a.gscale, a.ids, a.x, a.x_per_slot, a.y, a.experts, a.n,
                           a.k, pairs, a.topk, round_cap);
    else
        hipLaunchKernelGGL((moe_kernel<FMT, CB, G, S, R, false>), dim3((unsigned)tiles, (unsigned)pairs),
                           dim3(kThreads), 0, st, a.codes, a.scales, a.gscale, a.ids, a.x, a.x_per_slot, a.y,
                           a.experts, a.n, a.k, pairs, a.topk, round_cap);
}

// Tile shape: lanes per row (g), k split (s), rows per lane (r), from the
// MI355X measurements: rows of >= 64 chunks take 16 lanes and 2 rows per
// lane; shorter rows take 8 lanes at one token and 4 lanes for more tokens
// (more rows per workgroup for the same activations).  MXQ_MOE_ROWS="g,s,r"
// overrides the choice (used only to compare variants when tuning).
template <int FMT, int CB>
static bool launch_moe_cb(const MoeArgs& a, hipStream_t st) {
    const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
    int g = 16, sp = 1, r = 2;
    if (nchunks < 64) {
        r = 1;
        g = (a.tokens == 1 && nchunks >= 8) ? 8 : 4;
    }
    if (const char* env = std::getenv("MXQ_MOE_ROWS")) std::sscanf(env, "%d,%d,%d", &g, &sp, &r);
#define MXQ_MOE_CASE(G_, S_, R_)                        \
    if (g == G_ && sp == S_ && r == R_) {              \
        launch_moe_inst<FMT, CB, G_, S_, R_>(a, st);   \
        return true;                                   \
    }
    MXQ_MOE_SHAPES(MXQ_MOE_CASE)
#undef MXQ_MOE_CASE
    return false;
}

bool launch_moe(const MoeArgs& a, hipStream_t st) {
    const bool wide = (code_bytes_per_row(a.fmt, a.k) % 16) == 0;
    switch (a.fmt) {
        case kMXFP4: return launch_moe_cb<kMXFP4, 16>(a, st);
        case kMXFP8: return launch_moe_cb<kMXFP8, 16>(a, st);
        case kNVFP4: return wide ? launch_moe_cb<kNVFP4, 16>(a, st) : launch_moe_cb<kNVFP4, 8>(a, st);
    }
    return false;
}

}  // namespace mxq
