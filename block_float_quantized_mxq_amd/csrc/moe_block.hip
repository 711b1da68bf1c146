// moe_block.hip -- the MoE decode block around the expert-indexed GEMV:
// routing (softmax top-k over router logits) and the down projection that
// consumes the gate/up outputs through SwiGLU and combines a token's routed
// experts with their routing weights.
//
// The "affine MoE" row of the ROCm status table in the "Build from source"
// manual runs single-token MoE decode as a fused two-kernel path, gate-up then
// down; slide 13 of the talk lists that port.  Here the two kernels are:
//
//  * the expert-indexed gate/up GEMV (moe_impl.hpp, every routed expert read
//    once) in its paired-row mode: each lane holds gate row j and up row j of
//    one expert, and the tile's end writes both outputs and the activation
//    a_s[j] = bf16(silu(gate) * up) (fp32, rounded to nearest even once);
//  * moe_down_kernel below, grid (row tile of the hidden dimension, token): a
//    workgroup copies the token's topk activation vectors into LDS, then
//    streams, for each of its output rows, the rows of the topk routed down
//    matrices: group s of each row set reads expert ids[t][s] (the streaming
//    engine's per-slot mode) and the groups' sums are combined with the
//    routing weights in a fixed order -- no atomics, bit-reproducible.
//  * a token with an expert id outside [0, E) gets NaN outputs.
//
// Routing: one wave per token.  Selection compares the fp32 logits
// themselves (larger first, equal logits: lower index first), so it does not
// depend on how the softmax is rounded; the weights are the softmax
// probabilities of the selected experts, optionally renormalised over them.
#include <cstdlib>
#include <mutex>

#include "kernels.hpp"
#include "moe_route.hpp"
#include "rows_core.hpp"

namespace mxq {

// ---- routing ---------------------------------------------------------------------

template <int NS>
__global__ __launch_bounds__(64) void moe_route_kernel(const float* __restrict__ logits, int64_t experts,
                                                        int topk, int renorm, int32_t* __restrict__ ids,
                                                        float* __restrict__ weights) {
    const int64_t t = blockIdx.x;
    route_wave<NS>(logits + t * experts, (int)experts, topk, renorm, ids + t * topk, weights + t * topk);
}

template <int NS>
static void launch_route_ns(const RouteArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(moe_route_kernel<NS>, dim3((unsigned)a.tokens), dim3(64), 0, st, a.logits, a.experts,
                       (int)a.topk, a.renorm, a.ids, a.weights);
}

bool launch_moe_route(const RouteArgs& a, hipStream_t st) {
    if (a.experts > kRouteMaxExperts) return false;
    // logits per lane: the smallest compiled count that covers the experts
    if (a.experts <= 64) launch_route_ns<1>(a, st);
    else if (a.experts <= 128) launch_route_ns<2>(a, st);
    else if (a.experts <= 256) launch_route_ns<4>(a, st);
    else if (a.experts <= 512) launch_route_ns<8>(a, st);
    else launch_route_ns<kRouteSlots>(a, st);
    return true;
}

// ---- down projection with SwiGLU input and weighted combine ---------------------------

template <int FMT, int CB, int G, int S, int R>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gscale,
                                                            const int32_t* __restrict__ ids,
                                                            const float* __restrict__ weights,
                                                            const uint16_t* __restrict__ act, float* __restrict__ y,
                                                            int64_t experts, int64_t hidden, int64_t dff, int topk) {
    using T = RowTile<G, S, R>;
    using E = RowEngine<FMT, CB, 1, G, S, R, true, true>;
    using CS = ChunkShape<FMT, CB>;
    __shared__ float red[S > 1 ? S * T::ROWSETS * R : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
    const int64_t t = blockIdx.y;
    const int64_t row0 = (int64_t)blockIdx.x * T::ROWS;

    // routing of token t: multipliers (weight times the NVFP4 tensor scale)
    float smul[S];
    bool ok = true;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        smul[s] = 0.0f;
        if (s < topk) {
            const int e = ids[t * topk + s];
            ok = ok && e >= 0 && (int64_t)e < experts;
            const float gs = (FMT == kNVFP4 && e >= 0 && (int64_t)e < experts) ? gscale[e] : 1.0f;
            smul[s] = weights[t * topk + s] * gs;
        }
    }
    if (!ok) {
        for (int r = threadIdx.x; r < T::ROWS; r += kThreads)
            if (row0 + r < hidden) y[t * hidden + row0 + r] = __builtin_nanf("");
        return;
    }
    // this lane's group streams the down matrix of slot sp (slots past topk
    // repeat slot 0 and are left out of the combine)
    const int sp = (threadIdx.x / G) % S;
    const int e = ids[t * topk + (sp < topk ? sp : 0)];
    const int64_t rowbytes = code_bytes_per_row(FMT, dff);
    const E eng(codes + (int64_t)e * hidden * rowbytes, scales + (int64_t)e * hidden * (dff / CS::BS), hidden, dff);
    const uint16_t* xs[1] = {act};
    float* ys[1] = {y + t * hidden};
    RowCursor<R> cur = eng.cursor(row0, 0, 1, xs[0]);
    PassRing<RowPass<FMT, CB, R>, 2> ring;
    eng.template prime<1>(cur, ring);  // weights first: in flight while the activations are built

    // the token's activations [topk][dff] (slot s at elements s*dff ..) into
    // the staged block, 16 bytes a piece; the loads of U pieces per thread
    // are issued together (one cache round trip per U pieces)
    constexpr int U = 4;
    const int64_t pieces = (int64_t)topk * dff / 8;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(act + t * topk * dff);
    for (int64_t p0 = threadIdx.x; p0 < pieces; p0 += U * kThreads) {
        u32x4_t v[U];
#pragma unroll
        for (int w = 0; w < U; ++w) {
            const int64_t p = p0 + (int64_t)w * kThreads;
            v[w] = src[p < pieces ? p : p0];
        }
#pragma unroll
        for (int w = 0; w < U; ++w) {
            const int64_t p = p0 + (int64_t)w * kThreads;
            if (p < pieces) {
                const int64_t c = p / CS::XQ;
                const int q = (int)(p % CS::XQ);
                reinterpret_cast<u32x4_t*>(xlds)[c * CS::XQ + (q ^ x_swizzle<FMT, CB>(c))] = v[w];
            }
        }
    }
    lds_barrier();
    eng.template run<1>(cur, ring, xs, ys, 1.0f, red, xlds, smul, topk);
}

template <int FMT, int CB, int G, int S, int R>
static void launch_down_inst(const MoeBlockArgs& a, hipStream_t st) {
    using T = RowTile<G, S, R>;
    const int64_t tiles = (a.hidden + T::ROWS - 1) / T::ROWS;
    const size_t lds = (size_t)S * a.dff * 2;
    hipLaunchKernelGGL((moe_down_kernel<FMT, CB, G, S, R>), dim3((unsigned)tiles, (unsigned)a.tokens), dim3(kThreads),
                       lds, st, a.dn_codes, a.dn_scales, a.dn_gscale, a.ids, a.weights, a.act, a.y, a.experts, a.hidden,
                       a.dff, (int)a.topk);
}

// Two rows per lane at every token count: with the activations precomputed
// by the gate/up kernel, 4 rows per lane (half the workgroups, each copying
// its token's activations once) measure the same (MI355X, 30B-A3B block,
// 2 and 4 tokens: 17.89 / 25.70 us with 4, 17.89 / 25.76 us with 2) and
// one token is faster with 2 (14.74 vs 15.00 us); one row per lane (twice the
// workgroups) is slower at every token count (routed block, 1 / 2 / 4 tokens:
// 13.96 / 17.01 / 27.67 us against 13.47 / 16.48 / 26.43 us).
template <int FMT, int CB, int G, int S>
static void launch_down_gs(const MoeBlockArgs& a, hipStream_t st) {
    launch_down_inst<FMT, CB, G, S, 2>(a, st);
}

// Slots rounded up to a power of two; 8 lanes per row while a slot's row has
// at most 32 chunks, else 16.
template <int FMT, int CB>
static bool launch_down_cb(const MoeBlockArgs& a, hipStream_t st) {
    const int64_t chunks = code_bytes_per_row(FMT, a.dff) / CB;
    const bool narrow = chunks <= 32;
    switch (a.topk <= 1 ? 1 : a.topk <= 2 ? 2 : a.topk <= 4 ? 4 : a.topk <= 8 ? 8 : 16) {
        case 1: narrow ? launch_down_gs<FMT, CB, 8, 1>(a, st) : launch_down_gs<FMT, CB, 16, 1>(a, st); return true;
        case 2: narrow ? launch_down_gs<FMT, CB, 8, 2>(a, st) : launch_down_gs<FMT, CB, 16, 2>(a, st); return true;
        case 4: narrow ? launch_down_gs<FMT, CB, 8, 4>(a, st) : launch_down_gs<FMT, CB, 16, 4>(a, st); return true;
        case 8: narrow ? launch_down_gs<FMT, CB, 8, 8>(a, st) : launch_down_gs<FMT, CB, 16, 8>(a, st); return true;
        default: narrow ? launch_down_gs<FMT, CB, 8, 16>(a, st) : launch_down_gs<FMT, CB, 16, 16>(a, st); return true;
    }
}

bool launch_moe_down(const MoeBlockArgs& a, hipStream_t st) {
    // the staged activations of the padded slot count must fit the LDS budget
    const int64_t slots = a.topk <= 1 ? 1 : a.topk <= 2 ? 2 : a.topk <= 4 ? 4 : a.topk <= 8 ? 8 : 16;
    if (slots * a.dff * 2 > kMoeBlockMaxLds) return false;
    switch (a.fmt) {
        case kMXFP4: return launch_down_cb<kMXFP4, 16>(a, st);
        case kMXFP8: return launch_down_cb<kMXFP8, 16>(a, st);
        case kNVFP4:
            return (code_bytes_per_row(kNVFP4, a.dff) % 16) == 0 ? launch_down_cb<kNVFP4, 16>(a, st)
                                                                 : launch_down_cb<kNVFP4, 8>(a, st);
    }
    return false;
}

// ---- workspace of the allocation-free entry point -----------------------------------

// The gate/up outputs of mxq_moe_block_noalloc.  Host code never uses this
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device, and is cached below.  Every call on a device shares the
// array; h is written in full by the gate/up kernel before the down kernel
// reads it, so nothing needs clearing, and calls that overlap on one device
// (different streams) race on it.
static __device__ __align__(256) float scratch[kMoeBlockScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices];
}  // namespace

hipError_t moe_block_scratch(float** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace mxq
