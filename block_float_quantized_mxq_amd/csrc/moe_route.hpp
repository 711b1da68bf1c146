// moe_route.hpp -- top-k softmax routing of one token by one wave, shared by
// the routing kernel and the MoE gate/up kernel that routes in place.
//
// Selection compares the fp32 logits themselves (larger first, equal logits:
// lower index first), so it does not depend on how the softmax is rounded;
// the weights are the softmax probabilities of the selected experts,
// optionally renormalised over them.  Lanes l < topk of the wave write
// ids[l] and weights[l].
#pragma once

#include "mxq_device.hpp"

namespace mxq {

// Wave-uniform integer maximum and float sum: four DPP steps inside each row
// of 16 lanes, then the four row results are read into scalar registers and
// combined in a fixed order (row 0, 1, 2, 3), so every lane has the same bits.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ int wave_max_uniform(int v) {
    v = imax(v, dpp_i32<kDppQuadXor1>(v));
    v = imax(v, dpp_i32<kDppQuadXor2>(v));
    v = imax(v, dpp_i32<kDppRowHalfMirror>(v));
    v = imax(v, dpp_i32<kDppRowMirror>(v));
    return imax(imax(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                imax(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

__device__ __forceinline__ float wave_sum_uniform(float v) {
    v = group_sum<16>(v);
    const auto rl = [](float x, int lane) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
    };
    return ((rl(v, 0) + rl(v, 16)) + rl(v, 32)) + rl(v, 48);
}

// Order-preserving key of a float logit: signed-integer order of the keys is
// the order of the values (-0 is taken as +0, so equal values have equal
// keys); the inverse map is the same xor.
__device__ __forceinline__ int logit_key(float f) {
    int b = __builtin_bit_cast(int, f);
    b = b == (int)0x80000000 ? 0 : b;
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_logit(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF)); }

// One wave routes one token (any wave of a workgroup; lane l is its lane
// threadIdx.x % 64), everything in registers: lane l holds the keys of
// experts l, l + 64, ... (NS of them, at most 16).  Slot s gets the expert of
// rank s -- larger logit first, equal logits lower index first -- found in
// round s: the wave maximum m of the keys not yet picked, then the lowest
// index holding m, from one ballot per register slot (slot j holds experts
// 64 j .. 64 j + 63, so the first non-empty ballot and its lowest lane give
// the lowest index).  A picked expert's key becomes INT_MIN, below the key of
// every logit, -inf included, so -inf logits stay candidates.  The softmax
// maximum is round 0's winner; the probabilities are computed once, after the
// rounds, by the lanes l < topk, and the renormalising sum is a wave sum of
// them.  No LDS and no barrier.
constexpr int kRouteMaxExperts = 1024;
constexpr int kRouteSlots = kRouteMaxExperts / 64;

template <int NS>
__device__ __forceinline__ void route_wave(const float* __restrict__ lg, int E, int topk, int renorm,
                                           int32_t* __restrict__ ids, float* __restrict__ weights) {
    constexpr int kPicked = (int)0x80000000;
    const int l = threadIdx.x & 63;
    float v[NS];
    int key[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const bool in = l + 64 * j < E;
        v[j] = in ? lg[l + 64 * j] : 0.0f;
        key[j] = in ? logit_key(v[j]) : kPicked;
    }
    int top = kPicked, myk = kPicked, myi = -1;  // lane s ends with slot s's key and expert
    for (int s = 0; s < topk; ++s) {
        int m = key[0];
#pragma unroll
        for (int j = 1; j < NS; ++j) m = imax(m, key[j]);
        m = wave_max_uniform(m);
        int win = -1;
        if (m != kPicked) {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                if (win < 0) {
                    const uint64_t hit = __ballot(key[j] == m);
                    if (hit) {
                        const int lane = __builtin_ctzll(hit);
                        win = 64 * j + lane;
                        if (l == lane) key[j] = kPicked;
                    }
                }
            }
        }
        if (s == 0) top = m;
        if (l == s) {
            myk = m;
            myi = win;
        }
    }
    const float mx = key_logit(top);
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < NS; ++j)
        if (l + 64 * j < E) den += expf(v[j] - mx);
    den = wave_sum_uniform(den);
    const float p = l < topk ? expf(key_logit(myk) - mx) / den : 0.0f;
    const float psum = renorm ? wave_sum_uniform(p) : 1.0f;
    if (l < topk) {
        ids[l] = myi;
        weights[l] = renorm ? p / psum : p;
    }
}


}  // namespace mxq
