// moe_block.hip -- the MoE decode block around the expert-indexed GEMV:
// routing (softmax top-k over router logits) and the down projection that
// consumes the gate/up outputs through SwiGLU and combines a token's routed
// experts with their routing weights.
//
// The "affine MoE" row of the ROCm status table in the "Build from source"
// manual runs single-token MoE decode as a fused two-kernel path, gate-up then
// down; slide 13 of the talk lists that port.  Here the two kernels are the
// expert-indexed gate/up GEMV (moe_impl.hpp, every routed expert read once)
// and moe_down_kernel below:
//
//  * grid (row tile of the hidden dimension, token); a workgroup first turns
//    the token's gate/up outputs into its topk bf16 activation vectors
//    a_s = bf16(silu(gate) * up) in LDS (rounded to nearest even once), then
//    streams, for each of its output rows, the rows of the topk routed down
//    matrices: group s of each row set reads expert ids[t][s] (the streaming
//    engine's per-slot mode) and the groups' sums are combined with the
//    routing weights in a fixed order -- no atomics, bit-reproducible.
//  * a token with an expert id outside [0, E) gets NaN outputs.
//
// Routing: one workgroup per token.  Selection compares the fp32 logits
// themselves (larger first, equal logits: lower index first), so it does not
// depend on how the softmax is rounded; the weights are the softmax
// probabilities of the selected experts, optionally renormalised over them.
#include <cstdlib>
#include <mutex>

#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

// ---- routing ---------------------------------------------------------------------

__device__ __forceinline__ void take_better(float& v, int& i, float ov, int oi) {
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Largest (value, index) pair of the wave, equal values: lower index; every
// lane ends with it.  Inside each row of 16 lanes the partners come from DPP
// (swap neighbours, swap pairs, mirror halves, mirror the row: each step
// pairs every lane with one that holds the other half of its group), across
// rows from two shuffles.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    take_better(v, i, dpp_f32<kDppQuadXor1>(v), dpp_i32<kDppQuadXor1>(i));
    take_better(v, i, dpp_f32<kDppQuadXor2>(v), dpp_i32<kDppQuadXor2>(i));
    take_better(v, i, dpp_f32<kDppRowHalfMirror>(v), dpp_i32<kDppRowHalfMirror>(i));
    take_better(v, i, dpp_f32<kDppRowMirror>(v), dpp_i32<kDppRowMirror>(i));
    take_better(v, i, __shfl_xor(v, 16, 64), __shfl_xor(i, 16, 64));
    take_better(v, i, __shfl_xor(v, 32, 64), __shfl_xor(i, 32, 64));
}

// One workgroup per token.  The logits go to LDS; each expert's rank is the
// number of logits that beat it (larger, or equal with a lower index), so the
// selected experts are those of rank < topk and the rank is their output
// slot -- the same order as picking the largest remaining logit topk times,
// without topk serial rounds.  The softmax maximum and denominator are
// workgroup reductions; the renormalising sum adds the selected
// probabilities in slot order.
constexpr int kRouteThreads = 256;
constexpr int kRouteMaxExperts = 1024;

__device__ __forceinline__ float wave_max(float v) {
    int dummy = 0;
    wave_argmax(v, dummy);
    return v;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const float* __restrict__ logits, int64_t experts,
                                                                  int topk, int renorm, int32_t* __restrict__ ids,
                                                                  float* __restrict__ weights) {
    __shared__ __attribute__((aligned(16))) float lv[kRouteMaxExperts];
    __shared__ float part[kRouteThreads / 64];
    __shared__ float psel[16];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int E = (int)experts;
    const float* l = logits + t * experts;

    float mx = -__builtin_huge_valf();
    for (int e = tid; e < E; e += kRouteThreads) {
        const float v = l[e];
        lv[e] = v;
        mx = v > mx ? v : mx;
    }
    for (int e = E + tid; e < ((E + 15) & ~15); e += kRouteThreads) lv[e] = -__builtin_huge_valf();  // pad to 16
    mx = wave_max(mx);
    if ((tid & 63) == 0) part[wave] = mx;
    __syncthreads();
    mx = part[0];
#pragma unroll
    for (int w = 1; w < kRouteThreads / 64; ++w) mx = part[w] > mx ? part[w] : mx;
    __syncthreads();  // part is reused below

    float den = 0.0f;
    for (int e = tid; e < E; e += kRouteThreads) den += expf(lv[e] - mx);
    den = group_sum<64>(den);
    if ((tid & 63) == 0) part[wave] = den;
    __syncthreads();
    den = part[0];
#pragma unroll
    for (int w = 1; w < kRouteThreads / 64; ++w) den += part[w];

    for (int e = tid; e < E; e += kRouteThreads) {
        const float v = lv[e];
        // 16 logits per step: four independent LDS reads in flight (the
        // padding never counts: -inf beats nothing, and its index is past e)
        int rank = 0;
        for (int j0 = 0; j0 < E; j0 += 16) {
            float4 o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = *reinterpret_cast<const float4*>(lv + j0 + 4 * q);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + 4 * q;
                rank += (o[q].x > v || (o[q].x == v && j < e)) ? 1 : 0;
                rank += (o[q].y > v || (o[q].y == v && j + 1 < e)) ? 1 : 0;
                rank += (o[q].z > v || (o[q].z == v && j + 2 < e)) ? 1 : 0;
                rank += (o[q].w > v || (o[q].w == v && j + 3 < e)) ? 1 : 0;
            }
        }
        if (rank < topk) {
            ids[t * topk + rank] = e;
            psel[rank] = expf(v - mx) / den;
        }
    }
    __syncthreads();
    if (tid < topk) {
        float sel = 0.0f;
        for (int s = 0; s < topk; ++s) sel += psel[s];
        weights[t * topk + tid] = renorm ? psel[tid] / sel : psel[tid];
    }
}

bool launch_moe_route(const RouteArgs& a, hipStream_t st) {
    if (a.experts > kRouteMaxExperts) return false;
    hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)a.tokens), dim3(kRouteThreads), 0, st, a.logits, a.experts,
                       (int)a.topk, a.renorm, a.ids, a.weights);
    return true;
}

// ---- down projection with SwiGLU input and weighted combine ---------------------------

// a = bf16(silu(g) * u), computed in fp32 and rounded to nearest even once.
__device__ __forceinline__ uint32_t swiglu_bf16x2(float g0, float u0, float g1, float u1) {
    const float a0 = g0 / (1.0f + expf(-g0)) * u0;
    const float a1 = g1 / (1.0f + expf(-g1)) * u1;
    const bf16x2_t b = {(__bf16)a0, (__bf16)a1};
    return __builtin_bit_cast(uint32_t, b);
}

template <int FMT, int CB, int G, int S, int R>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gscale,
                                                            const int32_t* __restrict__ ids,
                                                            const float* __restrict__ weights,
                                                            const float* __restrict__ h, float* __restrict__ y,
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
    const uint16_t* xs[1] = {reinterpret_cast<const uint16_t*>(h)};
    float* ys[1] = {y + t * hidden};
    RowCursor<R> cur = eng.cursor(row0, 0, 1, xs[0]);
    PassRing<RowPass<FMT, CB, R>, 2> ring;
    eng.template prime<1>(cur, ring);  // weights first: in flight while the activations are built

    // activations of the token's slots, slot s at elements s*dff .. of the staged block
    // (the h loads of U pieces per thread are issued together: one cache
    // round trip per U pieces, not per piece)
    constexpr int U = 3;
    const int64_t pieces = (int64_t)topk * dff / 8;
    for (int64_t p0 = threadIdx.x; p0 < pieces; p0 += U * kThreads) {
        float4 g[U][2], u[U][2];
#pragma unroll
        for (int w = 0; w < U; ++w) {
            const int64_t p = p0 + (int64_t)w * kThreads;
            const int64_t pp = p < pieces ? p : p0;
            const int64_t s = pp * 8 / dff, j = pp * 8 % dff;
            const float* hg = h + (t * topk + s) * 2 * dff + j;
            g[w][0] = *reinterpret_cast<const float4*>(hg);
            g[w][1] = *reinterpret_cast<const float4*>(hg + 4);
            u[w][0] = *reinterpret_cast<const float4*>(hg + dff);
            u[w][1] = *reinterpret_cast<const float4*>(hg + dff + 4);
        }
#pragma unroll
        for (int w = 0; w < U; ++w) {
            const int64_t p = p0 + (int64_t)w * kThreads;
            if (p < pieces) {
                const float4 g0 = g[w][0], g1 = g[w][1], u0 = u[w][0], u1 = u[w][1];
                const u32x4_t v = {swiglu_bf16x2(g0.x, u0.x, g0.y, u0.y), swiglu_bf16x2(g0.z, u0.z, g0.w, u0.w),
                                   swiglu_bf16x2(g1.x, u1.x, g1.y, u1.y), swiglu_bf16x2(g1.z, u1.z, g1.w, u1.w)};
                const int64_t c = p / CS::XQ;
                const int q = (int)(p % CS::XQ);
                reinterpret_cast<u32x4_t*>(xlds)[c * CS::XQ + (q ^ x_swizzle<FMT, CB>(c))] = v;
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
                       lds, st, a.dn_codes, a.dn_scales, a.dn_gscale, a.ids, a.weights, a.h, a.y, a.experts, a.hidden,
                       a.dff, (int)a.topk);
}

// Rows per lane: a workgroup builds its token's activations once for all its
// rows, so from two tokens 4 rows per lane (half the workgroups, half the
// rebuilt activations) beat 2 (MI355X, 30B-A3B block: 4 tokens 33.0 -> 30.0 us,
// 8 tokens 49.6 -> 45.0 us; one token 18.0 vs 18.6 us, so 2 there).
template <int FMT, int CB, int G, int S>
static void launch_down_gs(const MoeBlockArgs& a, hipStream_t st) {
    if (a.tokens >= 2) launch_down_inst<FMT, CB, G, S, 4>(a, st);
    else launch_down_inst<FMT, CB, G, S, 2>(a, st);
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
