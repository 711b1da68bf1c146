// kernels.hpp -- host-side interface between the C ABI (api.hip) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.hpp"

namespace mxq {

struct GemvArgs {
    int fmt;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* gscale;
    const uint16_t* x;
    float* y;
    int64_t n, k, batch;
};

// Dense GEMV stream kernel settings: lanes per row (g), prefetch depth d
// (chunks in flight per lane), activations staged in LDS (xl), workgroups in
// the grid (wgs; rows are dealt round-robin over its groups).  The compiled
// (g, d) pairs are listed in MXQ_STREAM_SHAPES.
struct GemvConfig {
    int g, d, xl;
    int64_t wgs;
};

#define MXQ_STREAM_SHAPES(X) X(16, 4) X(32, 4) X(64, 4) X(64, 8)

struct MoeArgs {
    int fmt;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* gscale;
    const int32_t* ids;
    const uint16_t* x;
    int x_per_slot;
    float* y;
    int64_t experts, n, k, tokens, topk;
};

struct DequantArgs {
    int fmt;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* gscale;
    float* w;
    int64_t rows, k;
};

struct GemmArgs {
    int fmt;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* gscale;
    const uint16_t* x;
    void* y;
    int y_bf16;
    int64_t m, n, k;
};

GemvConfig choose_gemv_config(int fmt, int64_t n, int64_t k, int64_t batch);
bool launch_gemv(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st);
bool launch_moe(const MoeArgs& a, hipStream_t st);
bool launch_dequant(const DequantArgs& a, hipStream_t st);
bool launch_gemm(const GemmArgs& a, hipStream_t st);

}  // namespace mxq
