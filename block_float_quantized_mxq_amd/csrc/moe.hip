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
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

constexpr int kMaxPairs = 8 * 16;  // MXQ_MAX_BATCH * MXQ_MAX_TOPK

template <int FMT, int CB, int B, int G, int R>
__device__ __forceinline__ void moe_batch(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                          int64_t row0, const int* sel, int cnt, const uint16_t* x,
                                          int x_per_slot, int64_t topk, float* y, float gmul) {
    const uint16_t* xs[B];
    float* ys[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int q = sel[b < cnt ? b : 0];
        const int64_t xrow = x_per_slot ? (int64_t)q : (int64_t)q / topk;
        xs[b] = x + xrow * k;
        ys[b] = b < cnt ? y + (int64_t)q * n : nullptr;
    }
    rows_core<FMT, CB, B, G, 1, R, false>(codes, scales, n, k, row0, xs, ys, gmul, nullptr, nullptr);
}

template <int FMT, int CB, int G, int R>
__global__ __launch_bounds__(kThreads) void moe_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ gscale,
                                                       const int32_t* __restrict__ ids,
                                                       const uint16_t* __restrict__ x, int x_per_slot,
                                                       float* __restrict__ y, int64_t experts, int64_t n, int64_t k,
                                                       int pairs, int64_t topk) {
    using T = RowTile<G, 1, R>;
    __shared__ int sel[kMaxPairs];
    __shared__ int nsel;
    const int p = blockIdx.y;
    const int64_t row0 = (int64_t)blockIdx.x * T::ROWS;
    const int e = ids[p];
    if (e < 0 || (int64_t)e >= experts) {
        for (int t = threadIdx.x; t < T::ROWS; t += kThreads)
            if (row0 + t < n) y[(int64_t)p * n + row0 + t] = __builtin_nanf("");
        return;
    }
    for (int q = 0; q < p; ++q)
        if (ids[q] == e) return;  // an earlier position streams this expert
    if (threadIdx.x == 0) {
        int c = 0;
        for (int q = p; q < pairs; ++q)
            if (ids[q] == e) sel[c++] = q;
        nsel = c;
    }
    __syncthreads();
    const int total = nsel;
    const int64_t rowbytes = code_bytes_per_row(FMT, k);
    const uint8_t* ecodes = codes + (int64_t)e * n * rowbytes;
    const uint8_t* escales = scales + (int64_t)e * n * (k / BlockSize<FMT>::value);
    const float gmul = (FMT == kNVFP4) ? gscale[e] : 1.0f;
    for (int base = 0; base < total; base += 8) {
        const int cnt = total - base < 8 ? total - base : 8;
        const int* s = sel + base;
        if (cnt == 1) moe_batch<FMT, CB, 1, G, R>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul);
        else if (cnt == 2) moe_batch<FMT, CB, 2, G, R>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul);
        else if (cnt <= 4) moe_batch<FMT, CB, 4, G, R>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul);
        else moe_batch<FMT, CB, 8, G, R>(ecodes, escales, n, k, row0, s, cnt, x, x_per_slot, topk, y, gmul);
    }
}

template <int FMT, int CB, int G, int R>
static void launch_moe_inst(const MoeArgs& a, hipStream_t st) {
    using T = RowTile<G, 1, R>;
    const int64_t tiles = (a.n + T::ROWS - 1) / T::ROWS;
    const int pairs = (int)(a.tokens * a.topk);
    hipLaunchKernelGGL((moe_kernel<FMT, CB, G, R>), dim3((unsigned)tiles, (unsigned)pairs), dim3(kThreads), 0, st,
                       a.codes, a.scales, a.gscale, a.ids, a.x, a.x_per_slot, a.y, a.experts, a.n, a.k, pairs, a.topk);
}

template <int FMT, int CB>
static void launch_moe_cb(const MoeArgs& a, hipStream_t st) {
    // Lanes per row: as many as keep every lane busy on at least two chunks.
    const int64_t nchunks = code_bytes_per_row(FMT, a.k) / CB;
    if (nchunks >= 32) launch_moe_inst<FMT, CB, 16, 1>(a, st);
    else if (nchunks >= 16) launch_moe_inst<FMT, CB, 8, 1>(a, st);
    else launch_moe_inst<FMT, CB, 4, 1>(a, st);
}

bool launch_moe(const MoeArgs& a, hipStream_t st) {
    const bool wide = (code_bytes_per_row(a.fmt, a.k) % 16) == 0;
    switch (a.fmt) {
        case kMXFP4: launch_moe_cb<kMXFP4, 16>(a, st); return true;
        case kMXFP8: launch_moe_cb<kMXFP8, 16>(a, st); return true;
        case kNVFP4:
            if (wide) launch_moe_cb<kNVFP4, 16>(a, st);
            else launch_moe_cb<kNVFP4, 8>(a, st);
            return true;
    }
    return false;
}

}  // namespace mxq
