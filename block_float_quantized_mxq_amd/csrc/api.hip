// api.hip -- the C ABI declared in include/mxq.h: host-side validation, the
// gfx950 device check, kernel-configuration choice and launch.
//
// Validation happens before any HIP call, so argument errors are reported on
// machines without a GPU as well.  Checks run in the order the header lists
// (format, null pointers, shapes, alignment, supported sizes, device).
#include <atomic>
#include <cstring>

#include "../../include/mxq.h"
#include "kernels.hpp"

#define MXQ_API extern "C" __attribute__((visibility("default")))

namespace {

using mxq::kMXFP4;
using mxq::kMXFP8;
using mxq::kNVFP4;

bool valid_fmt(int fmt) { return fmt == kMXFP4 || fmt == kMXFP8 || fmt == kNVFP4; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Prefill GEMMs with at most this many token rows run on the matrix-unit GEMV
// (16 rows per launch).
constexpr int64_t kSmallGemmRows = 32;

// Per-device result of the gfx950 check: 0 unknown, 1 ok, 2 not usable; and
// the device's compute-unit count.
std::atomic<int> g_device_ok[64];
std::atomic<int> g_device_cus[64];

// gfx950 check of the current device; on success *cus is its compute-unit count.
mxq_status_t check_device(int* cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return MXQ_E_DEVICE;
    }
    if (dev >= 64) return MXQ_E_DEVICE;
    int state = g_device_ok[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return MXQ_E_DEVICE;
        }
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1, std::memory_order_relaxed);
        g_device_ok[dev].store(state, std::memory_order_release);
    }
    if (state != 1) return MXQ_E_DEVICE;
    *cus = g_device_cus[dev].load(std::memory_order_relaxed);
    return MXQ_OK;
}

mxq_status_t check_weight(int fmt, const uint8_t* codes, const uint8_t* scales, const float* gscale) {
    if (!valid_fmt(fmt)) return MXQ_E_FORMAT;
    if ((fmt == kNVFP4) != (gscale != nullptr)) return MXQ_E_FORMAT;
    if (!codes || !scales) return MXQ_E_NULLPTR;
    return MXQ_OK;
}

mxq_status_t check_k(int fmt, int64_t k) {
    if (k <= 0 || k % mxq::block_elems(fmt) != 0) return MXQ_E_SHAPE;
    return MXQ_OK;
}

mxq_status_t launched(bool ok) {
    if (!ok) return MXQ_E_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_E_LAUNCH;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace


MXQ_API const char* mxq_status_string(int s) {
    switch (s) {
        case MXQ_OK: return "ok";
        case MXQ_E_NULLPTR: return "a required pointer is NULL";
        case MXQ_E_SHAPE: return "invalid size (non-positive, or k not a multiple of the block size)";
        case MXQ_E_ALIGN: return "pointer not aligned (codes/activations 16 bytes, outputs/ids/scale 4 bytes)";
        case MXQ_E_FORMAT: return "invalid format, output type, or global_scale presence";
        case MXQ_E_UNSUPPORTED: return "size above the supported maximum";
        case MXQ_E_DEVICE: return "current device is not a gfx950 GPU";
        case MXQ_E_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

MXQ_API int mxq_abi_version(void) { return 9; }

MXQ_API mxq_status_t mxq_gemv(mxq_format_t fmt, const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                              const uint16_t* x, float* y, int64_t n, int64_t k, int64_t batch, void* stream) {
    mxq_status_t st = check_weight(fmt, codes, scales, global_scale);
    if (st != MXQ_OK) return st;
    if (!x || !y) return MXQ_E_NULLPTR;
    if (n <= 0 || batch <= 0) return MXQ_E_SHAPE;
    if ((st = check_k(fmt, k)) != MXQ_OK) return st;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(global_scale, 4)) return MXQ_E_ALIGN;
    if (n > kMaxDim || k > kMaxDim || batch > MXQ_MAX_BATCH) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const mxq::GemvArgs a{fmt, codes, scales, global_scale, x, y, n, k, batch, cus};
    return launched(mxq::launch_gemv(a, mxq::GemvConfig{}, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_gemv_config(mxq_format_t fmt, const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                                     const uint16_t* x, float* y, int64_t n, int64_t k, int64_t batch,
                                     const mxq_gemv_config_t* config, void* stream) {
    mxq_status_t st = check_weight(fmt, codes, scales, global_scale);
    if (st != MXQ_OK) return st;
    if (!x || !y || !config) return MXQ_E_NULLPTR;
    if (n <= 0 || batch <= 0) return MXQ_E_SHAPE;
    if ((st = check_k(fmt, k)) != MXQ_OK) return st;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(global_scale, 4)) return MXQ_E_ALIGN;
    if (n > kMaxDim || k > kMaxDim || batch > MXQ_MAX_BATCH) return MXQ_E_UNSUPPORTED;
    const mxq_gemv_config_t& c = *config;
    const int32_t fields[] = {c.rows_g, c.rows_s, c.rows_r, c.mm_r, c.mm_s, c.mfma_r, c.mfma_ks, c.mfma_nw, c.per_cu};
    for (int32_t f : fields)
        if (f < 0 || f > 64) return MXQ_E_UNSUPPORTED;
    if (c.grid < 0 || c.grid > 3) return MXQ_E_UNSUPPORTED;
    if (c.path != 0 && c.path != 1 && c.path != 2 && c.path != 4) return MXQ_E_UNSUPPORTED;
    if (c.path == 4 && batch > 4) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    mxq::GemvConfig cfg;
    cfg.path = c.path;
    cfg.rows_g = c.rows_g;
    cfg.rows_s = c.rows_s;
    cfg.rows_r = c.rows_r;
    cfg.rows_occ = c.per_cu;
    cfg.rows_grid = c.grid;
    cfg.mm_r = c.mm_r;
    cfg.mm_s = c.mm_s;
    cfg.mfma_r = c.mfma_r;
    cfg.mfma_ks = c.mfma_ks;
    cfg.mfma_nw = c.mfma_nw;
    cfg.mfma_occ = c.per_cu;
    const mxq::GemvArgs a{fmt, codes, scales, global_scale, x, y, n, k, batch, cus};
    return launched(mxq::launch_gemv(a, cfg, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_moe_gemv(mxq_format_t fmt, const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                                  const int32_t* expert_ids, const uint16_t* x, int x_per_slot, float* y,
                                  int64_t num_experts, int64_t n, int64_t k, int64_t tokens, int64_t topk,
                                  void* stream) {
    mxq_status_t st = check_weight(fmt, codes, scales, global_scale);
    if (st != MXQ_OK) return st;
    if (!expert_ids || !x || !y) return MXQ_E_NULLPTR;
    if (num_experts <= 0 || n <= 0 || tokens <= 0 || topk <= 0) return MXQ_E_SHAPE;
    if ((st = check_k(fmt, k)) != MXQ_OK) return st;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(expert_ids, 4) ||
        !aligned(global_scale, 4))
        return MXQ_E_ALIGN;
    if (n > kMaxDim || k > kMaxDim || num_experts > kMaxDim || tokens > MXQ_MAX_BATCH || topk > MXQ_MAX_TOPK)
        return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const mxq::MoeArgs a{fmt, codes, scales, global_scale, expert_ids, x, x_per_slot ? 1 : 0, y,
                         num_experts, n, k, tokens, topk, cus};
    return launched(mxq::launch_moe(a, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_gemm(mxq_format_t fmt, const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                              const uint16_t* x, void* y, mxq_out_t y_dtype, int64_t m, int64_t n, int64_t k,
                              void* stream) {
    mxq_status_t st = check_weight(fmt, codes, scales, global_scale);
    if (st != MXQ_OK) return st;
    if (y_dtype != MXQ_OUT_F32 && y_dtype != MXQ_OUT_BF16) return MXQ_E_FORMAT;
    if (!x || !y) return MXQ_E_NULLPTR;
    if (m <= 0 || n <= 0 || k <= 0) return MXQ_E_SHAPE;
    if ((st = check_k(fmt, k)) != MXQ_OK) return st;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(global_scale, 4)) return MXQ_E_ALIGN;
    if (m > kMaxDim || n > kMaxDim || k > kMaxDim) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    // (the matrix-unit GEMV takes whole 32-element blocks: an NVFP4 k that is an
    // odd multiple of 16 runs on the tiles at every m)
    if (m <= kSmallGemmRows && k % 32 == 0) {
        // Few token rows: the matrix-unit GEMV with one B-operand column per
        // row streams W once per 16 rows (MI355X, 25600 x 5120: 30-50 us for
        // 1-16 rows, 90-100 us for 24-32, against 138-146 us for the 256 x 256
        // tiles, whose 100 workgroups leave most of the GPU idle).  Both
        // output types take this path, so the bf16 output stays the RNE of the
        // fp32 one.
        const int64_t esz = y_dtype == MXQ_OUT_BF16 ? 2 : 4;
        for (int64_t r0 = 0; r0 < m; r0 += 16) {
            const int64_t rows = m - r0 < 16 ? m - r0 : 16;
            float* ys = reinterpret_cast<float*>(static_cast<uint8_t*>(y) + r0 * n * esz);
            mxq::GemvArgs g{fmt, codes, scales, global_scale, x + r0 * k, ys, n, k, rows, cus};
            g.y_bf16 = y_dtype == MXQ_OUT_BF16 ? 1 : 0;
            mxq::GemvConfig cfg;
            cfg.path = 1;
            if ((st = launched(mxq::launch_gemv(g, cfg, as_stream(stream)))) != MXQ_OK) return st;
        }
        return MXQ_OK;
    }
    const mxq::GemmArgs a{fmt, codes, scales, global_scale, x, y, y_dtype == MXQ_OUT_BF16 ? 1 : 0, m, n, k, cus};
    return launched(mxq::launch_gemm(a, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_dequant(mxq_format_t fmt, const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                                 float* w, int64_t rows, int64_t k, void* stream) {
    mxq_status_t st = check_weight(fmt, codes, scales, global_scale);
    if (st != MXQ_OK) return st;
    if (!w) return MXQ_E_NULLPTR;
    if (rows <= 0) return MXQ_E_SHAPE;
    if ((st = check_k(fmt, k)) != MXQ_OK) return st;
    if (!aligned(codes, 16) || !aligned(w, 4) || !aligned(global_scale, 4)) return MXQ_E_ALIGN;
    if (rows > kMaxDim || k > kMaxDim) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const mxq::DequantArgs a{fmt, codes, scales, global_scale, w, rows, k};
    return launched(mxq::launch_dequant(a, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_moe_route(const float* logits, int32_t* expert_ids, float* weights, int64_t tokens,
                                   int64_t num_experts, int64_t topk, int renorm, void* stream) {
    if (!logits || !expert_ids || !weights) return MXQ_E_NULLPTR;
    if (tokens <= 0 || num_experts <= 0 || topk <= 0 || topk > num_experts) return MXQ_E_SHAPE;
    if (!aligned(logits, 4) || !aligned(expert_ids, 4) || !aligned(weights, 4)) return MXQ_E_ALIGN;
    if (tokens > MXQ_MAX_BATCH || topk > MXQ_MAX_TOPK || num_experts > 1024) return MXQ_E_UNSUPPORTED;
    mxq_status_t st;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const mxq::RouteArgs a{logits, expert_ids, weights, tokens, num_experts, topk, renorm ? 1 : 0};
    return launched(mxq::launch_moe_route(a, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_quantize(mxq_format_t fmt, const uint16_t* x, const float* global_scale, uint8_t* codes,
                                  uint8_t* scales, int64_t rows, int64_t k, void* stream) {
    if (fmt != MXQ_FMT_MXFP4 && fmt != MXQ_FMT_MXFP8 && fmt != MXQ_FMT_NVFP4) return MXQ_E_FORMAT;
    if ((fmt == MXQ_FMT_NVFP4) != (global_scale != nullptr)) return MXQ_E_FORMAT;
    if (!x || !codes || !scales) return MXQ_E_NULLPTR;
    if (rows <= 0) return MXQ_E_SHAPE;
    mxq_status_t st;
    if ((st = check_k(fmt, k)) != MXQ_OK) return st;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(global_scale, 4)) return MXQ_E_ALIGN;
    if (rows > kMaxDim || k > kMaxDim || rows * k > mxq::kMaxQuantizeElems) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const mxq::QuantizeArgs a{fmt, x, global_scale, codes, scales, rows, k};
    return launched(mxq::launch_quantize(a, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_requant_fp8(const uint8_t* codes_in, const float* tile_scales, uint8_t* codes,
                                     uint8_t* scales, int64_t n, int64_t k, int64_t block_n, int64_t block_k,
                                     void* stream) {
    if (!codes_in || !tile_scales || !codes || !scales) return MXQ_E_NULLPTR;
    if (n <= 0 || k <= 0 || block_n <= 0 || block_k <= 0 || k % 32 != 0 || block_k % 32 != 0) return MXQ_E_SHAPE;
    if (!aligned(codes_in, 16) || !aligned(codes, 16) || !aligned(tile_scales, 4)) return MXQ_E_ALIGN;
    if (n > kMaxDim || k > kMaxDim || n * k > mxq::kMaxQuantizeElems) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    mxq_status_t st;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const mxq::RequantArgs a{codes_in, tile_scales, codes, scales, n, k, block_n, block_k};
    return launched(mxq::launch_requant_fp8(a, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_stream_read(const void* data, int64_t bytes, int layout, uint32_t* sink,
                                     int64_t sink_words, void* stream) {
    if (!data || !sink) return MXQ_E_NULLPTR;
    if (bytes <= 0 || bytes % 16 != 0 || sink_words <= 0) return MXQ_E_SHAPE;
    if (layout != 0 && layout != 1) return MXQ_E_FORMAT;
    if (!aligned(data, 16) || !aligned(sink, 4)) return MXQ_E_ALIGN;
    int cus = 0;
    mxq_status_t st;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const int64_t want = (int64_t)cus * mxq::kStreamReadPerCu;
    if (sink_words < want) return MXQ_E_UNSUPPORTED;
    return launched(mxq::launch_stream_read(data, bytes, sink, want, layout, as_stream(stream)));
}

MXQ_API mxq_status_t mxq_moe_gemm(mxq_format_t fmt, const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                                  const int32_t* expert_ids, const uint16_t* x, int x_per_slot, void* y,
                                  mxq_out_t y_dtype, int32_t* workspace, int64_t num_experts, int64_t m, int64_t n,
                                  int64_t k, int64_t topk, void* stream) {
    mxq_status_t st = check_weight(fmt, codes, scales, global_scale);
    if (st != MXQ_OK) return st;
    if (y_dtype != MXQ_OUT_F32 && y_dtype != MXQ_OUT_BF16) return MXQ_E_FORMAT;
    if (!expert_ids || !x || !y || !workspace) return MXQ_E_NULLPTR;
    if (num_experts <= 0 || m <= 0 || n <= 0 || k <= 0 || topk <= 0) return MXQ_E_SHAPE;
    if ((st = check_k(fmt, k)) != MXQ_OK) return st;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(global_scale, 4) ||
        !aligned(expert_ids, 4) || !aligned(workspace, 4))
        return MXQ_E_ALIGN;
    if (topk > MXQ_MAX_TOPK || num_experts > mxq::kMaxGroupExperts || m * topk > (int64_t(1) << 24) ||
        n > kMaxDim || k > kMaxDim)
        return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    const mxq::MoeGemmArgs a{fmt, codes, scales, global_scale, expert_ids, x, x_per_slot ? 1 : 0, y,
                             y_dtype == MXQ_OUT_BF16 ? 1 : 0, workspace, num_experts, m, n, k, topk};
    return launched(mxq::launch_moe_gemm(a, as_stream(stream)));
}

namespace {

// Validation of the MoE block's arguments, in the order the header lists; the
// workspace h is checked when need_h (the allocation-free variant has none).
mxq_status_t check_moe_block(int fmt, const uint8_t* gu_codes, const uint8_t* gu_scales, const float* gu_gscale,
                             const uint8_t* dn_codes, const uint8_t* dn_scales, const float* dn_gscale,
                             const int32_t* expert_ids, const float* weights, const uint16_t* x, const float* h,
                             bool need_h, const float* y, int64_t num_experts, int64_t hidden, int64_t dff,
                             int64_t tokens, int64_t topk) {
    mxq_status_t st = check_weight(fmt, gu_codes, gu_scales, gu_gscale);
    if (st != MXQ_OK) return st;
    if ((st = check_weight(fmt, dn_codes, dn_scales, dn_gscale)) != MXQ_OK) return st;
    if (!expert_ids || !weights || !x || (need_h && !h) || !y) return MXQ_E_NULLPTR;
    if (num_experts <= 0 || tokens <= 0 || topk <= 0) return MXQ_E_SHAPE;
    if ((st = check_k(fmt, hidden)) != MXQ_OK) return st;
    if ((st = check_k(fmt, dff)) != MXQ_OK) return st;
    if (!aligned(gu_codes, 16) || !aligned(dn_codes, 16) || !aligned(x, 16) || !aligned(h, 16) || !aligned(y, 4) ||
        !aligned(expert_ids, 4) || !aligned(weights, 4) || !aligned(gu_gscale, 4) || !aligned(dn_gscale, 4))
        return MXQ_E_ALIGN;
    if (hidden > kMaxDim || dff > kMaxDim || num_experts > kMaxDim || tokens > MXQ_MAX_BATCH || topk > MXQ_MAX_TOPK)
        return MXQ_E_UNSUPPORTED;
    const int64_t slots = topk <= 1 ? 1 : topk <= 2 ? 2 : topk <= 4 ? 4 : topk <= 8 ? 8 : 16;
    if (slots * dff * 2 > mxq::kMoeBlockMaxLds) return MXQ_E_UNSUPPORTED;
    return MXQ_OK;
}

// The block's two kernels on validated arguments, with the workspace at h.
// With logits set, the gate/up kernel routes in place and writes the ids and
// weights (expert_ids / weights are then its outputs).
mxq_status_t run_moe_block(int fmt, const uint8_t* gu_codes, const uint8_t* gu_scales, const float* gu_gscale,
                           const uint8_t* dn_codes, const uint8_t* dn_scales, const float* dn_gscale,
                           const int32_t* expert_ids, const float* weights, const uint16_t* x, float* h, float* y,
                           int64_t num_experts, int64_t hidden, int64_t dff, int64_t tokens, int64_t topk, int cus,
                           void* stream, const float* logits = nullptr, int renorm = 0) {
    mxq_status_t st;
    // workspace: gate/up outputs, then the bf16 activations
    uint16_t* act = reinterpret_cast<uint16_t*>(h + tokens * topk * 2 * dff);
    mxq::MoeArgs gu{fmt, gu_codes, gu_scales, gu_gscale, expert_ids, x, 0, h, num_experts, 2 * dff, hidden,
                    tokens, topk, cus};
    gu.act = act;
    if (logits) {
        gu.logits = logits;
        gu.renorm = renorm ? 1 : 0;
        gu.ids_out = const_cast<int32_t*>(expert_ids);
        gu.weights_out = const_cast<float*>(weights);
    }
    if ((st = launched(mxq::launch_moe(gu, as_stream(stream)))) != MXQ_OK) return st;
    const mxq::MoeBlockArgs dn{fmt, dn_codes, dn_scales, dn_gscale, expert_ids, weights, act, y, num_experts, hidden,
                               dff, tokens, topk};
    return launched(mxq::launch_moe_down(dn, as_stream(stream)));
}

}  // namespace

MXQ_API mxq_status_t mxq_moe_block(mxq_format_t fmt, const uint8_t* gu_codes, const uint8_t* gu_scales, const float* gu_gscale,
                                   const uint8_t* dn_codes, const uint8_t* dn_scales, const float* dn_gscale,
                                   const int32_t* expert_ids, const float* weights, const uint16_t* x, float* h,
                                   float* y, int64_t num_experts, int64_t hidden, int64_t dff, int64_t tokens,
                                   int64_t topk, void* stream) {
    mxq_status_t st = check_moe_block(fmt, gu_codes, gu_scales, gu_gscale, dn_codes, dn_scales, dn_gscale, expert_ids,
                                      weights, x, h, true, y, num_experts, hidden, dff, tokens, topk);
    if (st != MXQ_OK) return st;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    return run_moe_block(fmt, gu_codes, gu_scales, gu_gscale, dn_codes, dn_scales, dn_gscale, expert_ids, weights, x, h,
                         y, num_experts, hidden, dff, tokens, topk, cus, stream);
}

MXQ_API mxq_status_t mxq_moe_block_routed(mxq_format_t fmt, const uint8_t* gu_codes, const uint8_t* gu_scales,
                                          const float* gu_gscale, const uint8_t* dn_codes, const uint8_t* dn_scales,
                                          const float* dn_gscale, const float* logits, int renorm,
                                          int32_t* expert_ids, float* weights, const uint16_t* x, float* h, float* y,
                                          int64_t num_experts, int64_t hidden, int64_t dff, int64_t tokens,
                                          int64_t topk, void* stream) {
    mxq_status_t st = check_moe_block(fmt, gu_codes, gu_scales, gu_gscale, dn_codes, dn_scales, dn_gscale, expert_ids,
                                      weights, x, h, true, y, num_experts, hidden, dff, tokens, topk);
    if (st != MXQ_OK) return st;
    if (!logits) return MXQ_E_NULLPTR;
    if (topk > num_experts) return MXQ_E_SHAPE;
    if (!aligned(logits, 4)) return MXQ_E_ALIGN;
    if (num_experts > 1024) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    return run_moe_block(fmt, gu_codes, gu_scales, gu_gscale, dn_codes, dn_scales, dn_gscale, expert_ids, weights, x, h,
                         y, num_experts, hidden, dff, tokens, topk, cus, stream, logits, renorm);
}

MXQ_API mxq_status_t mxq_moe_block_noalloc(mxq_format_t fmt, const uint8_t* gu_codes, const uint8_t* gu_scales,
                                           const float* gu_gscale, const uint8_t* dn_codes, const uint8_t* dn_scales,
                                           const float* dn_gscale, const int32_t* expert_ids, const float* weights,
                                           const uint16_t* x, float* y, int64_t num_experts, int64_t hidden,
                                           int64_t dff, int64_t tokens, int64_t topk, void* stream) {
    mxq_status_t st = check_moe_block(fmt, gu_codes, gu_scales, gu_gscale, dn_codes, dn_scales, dn_gscale, expert_ids,
                                      weights, x, nullptr, false, y, num_experts, hidden, dff, tokens, topk);
    if (st != MXQ_OK) return st;
    if (mxq::moe_block_workspace_bytes(tokens, topk, dff) > mxq::kMoeBlockScratchBytes) return MXQ_E_UNSUPPORTED;
    int cus = 0;
    if ((st = check_device(&cus)) != MXQ_OK) return st;
    float* h = nullptr;
    if (mxq::moe_block_scratch(&h) != hipSuccess || !h) {
        (void)hipGetLastError();
        return MXQ_E_DEVICE;
    }
    return run_moe_block(fmt, gu_codes, gu_scales, gu_gscale, dn_codes, dn_scales, dn_gscale, expert_ids, weights, x, h,
                         y, num_experts, hidden, dff, tokens, topk, cus, stream);
}
