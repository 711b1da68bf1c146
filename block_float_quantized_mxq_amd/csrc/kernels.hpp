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
    int cus;         // compute units of the device
    int y_bf16 = 0;  // matrix-unit path only: y holds bf16 (RNE), not fp32
};

// Dense GEMV settings (0 = chosen from the shape).  FMA rows: lanes per row
// (rows_g), k split (rows_s), rows per lane (rows_r), workgroups per CU
// (rows_occ), grid mode (rows_grid); the compiled (g, s, r) combinations are
// listed in MXQ_ROWS_SHAPES.  Matrix-mode rows: four-row groups per lane
// (mm_r), k split across waves (mm_s).  Matrix-unit GEMV: row blocks per wave
// (mfma_r), k split (mfma_ks), waves per workgroup (mfma_nw), workgroups per
// CU (mfma_occ).  mxq_gemv_config fills these from the caller's request.
struct GemvConfig {
    int rows_g = 0, rows_s = 0, rows_r = 0, rows_occ = 0;
    // 0: min(tiles, resident), tiles interleaved; 1: equal tiles per workgroup; 2: one workgroup per
    // tile; 3: min(tiles, resident), one contiguous range of tiles per workgroup
    int rows_grid = 0;
    // Path: 0 = by batch (FMA rows at batch 1, matrix-mode rows at 2 .. 4,
    // matrix unit from 5), 1 = matrix unit, 2 = FMA rows, 4 = matrix-mode rows
    // (batch <= 4).
    int path = 0;
    int mm_r = 0, mm_s = 0;
    int mfma_r = 0, mfma_ks = 0, mfma_nw = 0, mfma_occ = 0;
};

#define MXQ_ROWS_SHAPES(X) \
    X(4, 1, 1) X(8, 1, 1) X(16, 1, 1) X(16, 2, 1) X(16, 4, 1) X(16, 8, 1) X(16, 1, 2) X(16, 2, 2) X(16, 4, 2) \
    X(16, 8, 2) X(16, 1, 4) X(16, 2, 4) X(16, 4, 4) X(16, 8, 4)

// Compiled MoE tile shapes (lanes per row, k split, rows per lane).
#define MXQ_MOE_SHAPES(X) X(4, 1, 1) X(8, 1, 1) X(16, 1, 1) X(16, 1, 2)

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
    int cus;  // compute units of the device
    // non-null: the rows are a SwiGLU layer's gate rows then up rows (n even),
    // and position q also gets bf16(silu(gate) * up) at act + q n/2
    uint16_t* act = nullptr;
    // non-null (with act): the kernel routes in place from router logits
    // [tokens][experts] and writes the ids and weights it used to ids_out and
    // weights_out (ids is then not read)
    const float* logits = nullptr;
    int renorm = 0;
    int32_t* ids_out = nullptr;
    float* weights_out = nullptr;
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
    int cus;  // compute units of the device
};

bool launch_gemv(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st);
bool launch_moe(const MoeArgs& a, hipStream_t st);

struct RouteArgs {
    const float* logits;
    int32_t* ids;
    float* weights;
    int64_t tokens, experts, topk;
    int renorm;
};

struct MoeBlockArgs {
    int fmt;
    const uint8_t* dn_codes;
    const uint8_t* dn_scales;
    const float* dn_gscale;
    const int32_t* ids;
    const float* weights;
    const uint16_t* act;  // bf16 SwiGLU activations [tokens][topk][dff]
    float* y;             // [tokens][hidden]
    int64_t experts, hidden, dff, tokens, topk;
};

// LDS budget of the down kernel's staged activations (slots rounded up to a
// power of two, dff bf16 each).
constexpr int64_t kMoeBlockMaxLds = 64 * 1024;

// The MoE block's workspace: the gate/up outputs (fp32 [tokens][topk][2 dff])
// followed by the activations (bf16 [tokens][topk][dff]), 10 bytes per
// (token, slot, expert-width column).
constexpr int64_t moe_block_workspace_bytes(int64_t tokens, int64_t topk, int64_t dff) {
    return tokens * topk * dff * 10;
}
// Allocation-free MoE block: the workspace lives in a static device array of
// this many bytes, one per GPU.  Every call the LDS budget admits fits
// (topk * dff <= 32768 and tokens <= 8 give at most 2.5 MiB).
constexpr int64_t kMoeBlockScratchBytes = int64_t(5) << 19;
// The array's device address on the current device (looked up once per device).
hipError_t moe_block_scratch(float** ptr);

// Expert-batched MoE GEMM: Y[q][:] = W[ids[q]] . X[q / topk] (or X[q] with
// x_per_slot) for the pairs q = token * topk + slot; workspace: the caller's
// scratch of experts + 1 + m * topk int32 (the streaming kernel needs none).
struct MoeGemmArgs {
    int fmt;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* gscale;
    const int32_t* ids;
    const uint16_t* x;
    int x_per_slot;
    void* y;
    int y_bf16;
    int32_t* workspace;
    int64_t experts, m, n, k, topk;
};
constexpr int kMaxGroupExperts = 1024;  // experts per bank of the expert-batched GEMM

// Quantizer: bf16 x[rows][k] -> codes and block scales (NVFP4: per-tensor scale gscale[0] given).
struct QuantizeArgs {
    int fmt;
    const uint16_t* x;
    const float* gscale;
    uint8_t* codes;
    uint8_t* scales;
    int64_t rows, k;
};
constexpr int64_t kMaxQuantizeElems = int64_t(1) << 36;

bool launch_quantize(const QuantizeArgs& a, hipStream_t st);

// FP8 block checkpoint (E4M3 codes [n][k], fp32 scale per bn x bk tile) -> MXFP8.
struct RequantArgs {
    const uint8_t* codes_in;
    const float* tile_scales;
    uint8_t* codes;
    uint8_t* scales;
    int64_t n, k, bn, bk;
};
bool launch_requant_fp8(const RequantArgs& a, hipStream_t st);

// Streaming read of `bytes` (a multiple of 16) on `workgroups` workgroups,
// lanes interleaved over the range or one contiguous range per workgroup;
// sink[w] receives workgroup w's fold of the words it read.
bool launch_stream_read(const void* p, int64_t bytes, uint32_t* sink, int64_t workgroups, int contiguous,
                        hipStream_t st);
// Workgroups of the streaming read: as many as are resident on the device.
constexpr int kStreamReadPerCu = 8;
bool launch_moe_route(const RouteArgs& a, hipStream_t st);
bool launch_moe_gemm(const MoeGemmArgs& a, hipStream_t st);
bool launch_moe_down(const MoeBlockArgs& a, hipStream_t st);
bool launch_dequant(const DequantArgs& a, hipStream_t st);
bool launch_gemm(const GemmArgs& a, hipStream_t st);

}  // namespace mxq
