/*
 * mxq.h -- C ABI of libmxq: block-float quantized GEMV, expert-indexed MoE
 * GEMV and prefill GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation all entry points share is the one the "MLxcel 0.8 release"
 * post (backend.ai) describes in its section "Decoding block-float formats in
 * software", and slide 7 of the talk "High-performance LLM/VLM inference on
 * AMD Strix Halo with mlxcel engine" restates: weights stored as MXFP4, MXFP8
 * or NVFP4 blocks are unpacked to floating point inside the kernel and then
 * contracted with the activations.  Decode is exact (same section, and slide
 * 12 of the talk).  Decode speed is bounded by how fast the weights stream from
 * memory ("The memory wall" section of the post, slide 15 of the talk).
 *
 * Formats (OCP Microscaling v1.0 and NVFP4 public definitions; the pages give
 * the names and the E2M1 field widths only):
 *   MXFP4  32 E2M1 codes + one E8M0 block scale            (4.25 bits/weight)
 *   MXFP8  32 E4M3 codes (OCP "FN") + one E8M0 block scale (8.25 bits/weight)
 *   NVFP4  16 E2M1 codes + one E4M3 block scale, plus one fp32 scale per
 *          tensor (per expert in an MoE bank)                (4.5 bits/weight)
 *
 * Layout of a weight W[n][k] (n outputs, k the reduction dimension):
 *   codes  uint8 [n][k/2] for E2M1: byte j of a row holds element 2j in bits
 *          3:0 and element 2j+1 in bits 7:4;  uint8 [n][k] for E4M3.
 *   scales uint8 [n][k/32] (E8M0) or [n][k/16] (E4M3), row-major; block b of a
 *          row covers elements [b*bs, (b+1)*bs).
 *   An MoE bank stacks experts in front: [E][n][...].
 * Activations are bf16 bit patterns (uint16), row-major [rows][k].
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates and frees nothing and keeps no pointer after it returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  MXQ_OK means "validated and enqueued".
 *   - Arguments are validated on the host before anything is enqueued; the
 *     first failing check is returned and nothing runs:
 *       MXQ_E_FORMAT       unknown format, or global_scale given for an MX
 *                          format / missing for NVFP4, or unknown output type
 *       MXQ_E_NULLPTR      a required pointer is NULL
 *       MXQ_E_SHAPE        a size <= 0, or k not a multiple of the block size
 *                          (32 for MX formats, 16 for NVFP4)
 *       MXQ_E_ALIGN        codes or activations not 16-byte aligned, outputs,
 *                          expert ids or global_scale not 4-byte aligned
 *       MXQ_E_UNSUPPORTED  a size above the documented maximum
 *       MXQ_E_DEVICE       the current device is not a gfx950 GPU (or there is
 *                          no device)
 *       MXQ_E_LAUNCH       the kernel launch itself failed
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Offsets are computed in 64-bit arithmetic throughout.
 *   - Thread-safe and reentrant; no global mutable state besides a per-device
 *     capability cache filled once.  The library never prints.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     on every run (fixed reduction order, no atomics).
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats.  The parameters that take one are typed mxq_format_t, an
 * int, so that any value a caller passes is well defined on both sides of the
 * ABI; values outside the enumeration are rejected with MXQ_E_FORMAT. */
enum mxq_format { MXQ_FMT_MXFP4 = 1, MXQ_FMT_MXFP8 = 2, MXQ_FMT_NVFP4 = 3 };
typedef int mxq_format_t;

typedef enum {
    MXQ_OK = 0,
    MXQ_E_NULLPTR = 1,
    MXQ_E_SHAPE = 2,
    MXQ_E_ALIGN = 3,
    MXQ_E_FORMAT = 4,
    MXQ_E_UNSUPPORTED = 5,
    MXQ_E_DEVICE = 6,
    MXQ_E_LAUNCH = 7
} mxq_status_t;

/* Output element types of the GEMMs (an int for the same reason). */
enum mxq_out { MXQ_OUT_F32 = 0, MXQ_OUT_BF16 = 1 };
typedef int mxq_out_t;

/* Largest batch of the GEMV and largest token count of the MoE GEMV. */
#define MXQ_MAX_BATCH 8
/* Largest number of routed experts per token. */
#define MXQ_MAX_TOPK 16

/*
 * Dense GEMV (the decode projection; "Decoding block-float formats in
 * software" and "Profiling set the porting order" sections of the post, where
 * the quantized matrix-vector kernel takes 95% of dense decode time):
 *
 *   y[b][i] = sum_k W[i][k] * x[b][k]     for b < batch, i < n
 *
 * with W decoded exactly, products and sums in fp32, the NVFP4 per-tensor
 * scale applied once to each output.
 *   fmt           format of W
 *   codes, scales W as laid out above, n rows of k elements
 *   global_scale  NVFP4: pointer to one fp32 on the device; MX formats: NULL
 *   x             bf16 [batch][k]
 *   y             fp32 [batch][n] (written, never read)
 *   n, k          1 <= n, k < 2^31; k % block == 0
 *   batch         1 .. MXQ_MAX_BATCH
 */
mxq_status_t mxq_gemv(mxq_format_t fmt, const uint8_t *codes, const uint8_t *scales, const float *global_scale,
                      const uint16_t *x, float *y, int64_t n, int64_t k, int64_t batch, void *stream);

/*
 * Kernel configuration of the dense GEMV, for tests and tuning: the same
 * product as mxq_gemv with the kernel and its tile chosen by the caller
 * instead of from the shape.  Every field 0 means "chosen from the shape".
 *   path    0 by batch (FMA rows at batch 1, matrix-mode rows at 2..4, the
 *           matrix-unit GEMV from 5), 1 matrix-unit GEMV, 2 FMA rows,
 *           4 matrix-mode rows (batch <= 4)
 *   rows_g, rows_s, rows_r   FMA rows: lanes per row, k split, rows per lane
 *   mm_r, mm_s               matrix-mode rows: four-row groups per lane, k
 *                            split across waves
 *   mfma_r, mfma_ks, mfma_nw matrix-unit GEMV: row blocks per wave, k split,
 *                            waves per workgroup
 *   per_cu                   workgroups per compute unit
 *   grid                     FMA and matrix-mode rows: 0 as many workgroups as are resident,
 *                            tiles interleaved; 1 equal tile counts; 2 one
 *                            workgroup per tile; 3 as 0 with one contiguous
 *                            range of tiles per workgroup
 * A configuration that is not compiled returns MXQ_E_UNSUPPORTED and runs
 * nothing; config NULL is MXQ_E_NULLPTR.  Arguments as for mxq_gemv.
 */
typedef struct {
    int32_t path;
    int32_t rows_g, rows_s, rows_r;
    int32_t mm_r, mm_s;
    int32_t mfma_r, mfma_ks, mfma_nw;
    int32_t per_cu;
    int32_t grid;
} mxq_gemv_config_t;

mxq_status_t mxq_gemv_config(mxq_format_t fmt, const uint8_t *codes, const uint8_t *scales, const float *global_scale,
                             const uint16_t *x, float *y, int64_t n, int64_t k, int64_t batch,
                             const mxq_gemv_config_t *config, void *stream);

/*
 * Expert-indexed MoE GEMV: every routed (token, slot) pair multiplies its
 * activation vector by the weight of the expert it is routed to, and only the
 * routed experts' weights are read, each expert once per call however many
 * pairs route to it ("Unified memory" section of the post: a token reads only
 * its active experts; slide 4 of the talk).  No routing weights, no combine.
 *
 *   y[t][s][i] = sum_k W[ids[t][s]][i][k] * x_ts[k]
 *   x_ts = x[t]     (x_per_slot == 0: x is bf16 [tokens][k], e.g. gate/up)
 *   x_ts = x[t][s]  (x_per_slot != 0: x is bf16 [tokens][topk][k], e.g. down)
 *
 *   codes, scales  the bank: [num_experts][n][...]
 *   global_scale   NVFP4: fp32 [num_experts] on the device; MX: NULL
 *   expert_ids     int32 [tokens][topk] on the device.  Ids are not checked
 *                  on the host (that would need a synchronisation); a pair
 *                  whose id is outside [0, num_experts) gets a NaN output row.
 *   y              fp32 [tokens][topk][n]
 *   tokens         1 .. MXQ_MAX_BATCH;  topk 1 .. MXQ_MAX_TOPK
 */
mxq_status_t mxq_moe_gemv(mxq_format_t fmt, const uint8_t *codes, const uint8_t *scales, const float *global_scale,
                          const int32_t *expert_ids, const uint16_t *x, int x_per_slot, float *y,
                          int64_t num_experts, int64_t n, int64_t k, int64_t tokens, int64_t topk,
                          void *stream);

/*
 * Prefill GEMM on the same weights (compute bound; the post's "The memory
 * wall" section and slide 12 of the talk: decode to 16-bit floats on the GPU,
 * then the matrix unit):
 *
 *   Y[m][i] = sum_k X[m][k] * W[i][k]
 *
 * W is decoded to bf16 tiles and multiplied on the bf16 matrix cores with fp32
 * accumulation; the NVFP4 per-tensor scale multiplies the fp32 result.  The
 * decode is exact for every code at every scale byte: an E2M1 value times an
 * E8M0 scale is always a bf16 (subnormal, infinite or NaN included), so is an
 * E4M3 value at E8M0 bytes >= 3, and NVFP4's q * s has at most 6 significant
 * bits.  MXFP8 blocks with an E8M0 byte of 0, 1 or 2 (values finer than bf16's
 * smallest subnormal) are decoded 2^3 larger and their fp32 contribution is
 * multiplied by 2^-3, which is exact.
 *   x       bf16 [m][k]
 *   y       [m][n], fp32 (y_dtype MXQ_OUT_F32) or bf16 rounded to nearest even
 *           from the fp32 result (MXQ_OUT_BF16)
 *   m, n, k >= 1, < 2^31; k a multiple of the block size (32 MX, 16 NVFP4)
 * Up to 32 rows of X run on the matrix-unit GEMV (one B-operand column per
 * row) when k % 32 == 0; everything else on 256 x 256 output tiles.
 */
mxq_status_t mxq_gemm(mxq_format_t fmt, const uint8_t *codes, const uint8_t *scales, const float *global_scale,
                      const uint16_t *x, void *y, mxq_out_t y_dtype, int64_t m, int64_t n, int64_t k, void *stream);

/*
 * Decoded weights, for checking the in-kernel decode bit for bit:
 *   w[r][j] = fl32(q * 2^(u-127))        MX formats
 *   w[r][j] = fl32((q * s) * g)          NVFP4 (q*s is exact; one rounding)
 * with q the decoded code, u the E8M0 byte (255: NaN), s the decoded E4M3
 * block scale and g the per-tensor scale.  It runs the decode of the product
 * kernels: the scaled conversion with the E8M0 byte as its scale (MXFP8 bytes
 * 0..2 lifted by 2^3 and scaled back in fp32), or the unit-scale conversion
 * times s (NVFP4); the result is exact for every code and every scale byte.
 *   w   fp32 [rows][k]
 */
mxq_status_t mxq_dequant(mxq_format_t fmt, const uint8_t *codes, const uint8_t *scales, const float *global_scale,
                         float *w, int64_t rows, int64_t k, void *stream);

/*
 * MoE routing (the step before the expert-indexed GEMV in a decode block):
 * for each token t, the topk experts with the largest router logits are
 * selected, larger first, equal logits lower index first (the selection
 * compares the fp32 logits themselves, so it is exact); each gets its softmax
 * probability over all experts, divided by the sum of the selected ones when
 * `renorm` is nonzero.  Logits must not be NaN.
 *   logits   fp32 [tokens][num_experts], num_experts 1 .. 1024
 *   ids      int32 [tokens][topk] out;  weights fp32 [tokens][topk] out
 *   tokens   1 .. MXQ_MAX_BATCH;  topk 1 .. min(MXQ_MAX_TOPK, num_experts)
 */
mxq_status_t mxq_moe_route(const float *logits, int32_t *expert_ids, float *weights, int64_t tokens,
                           int64_t num_experts, int64_t topk, int renorm, void *stream);

/*
 * MoE decode block: the fused two-kernel path (gate/up, then down) that the
 * "affine MoE" row of the ROCm status table of the manual describes for
 * single-token decode:
 *
 *   h[t][s]    = W_gu[ids[t][s]] . x[t]                 (fp32, 2*dff outputs:
 *                                                       gate rows 0..dff-1,
 *                                                       up rows dff..2dff-1)
 *   a[t][s][j] = bf16(silu(h[t][s][j]) * h[t][s][dff+j]) silu(g) = g/(1+e^-g),
 *                                                       rounded to nearest even
 *   y[t][i]    = sum_s weights[t][s] * sum_j W_dn[ids[t][s]][i][j] * a[t][s][j]
 *
 * Kernel 1 is the expert-indexed GEMV of mxq_moe_gemv on the gate/up bank
 * (each routed expert read once) with gate row j and up row j in one lane: it
 * writes h and the activations a into the caller's workspace; kernel 2 copies
 * a token's activations into LDS and streams each output row of the token's
 * routed down matrices, combining them in a fixed order.  A token with an
 * expert id outside [0, num_experts) gets NaN outputs.
 *   gu_codes/gu_scales  gate/up bank [num_experts][2*dff][hidden] (layout as mxq_moe_gemv)
 *   dn_codes/dn_scales  down bank [num_experts][hidden][dff]
 *   gu_gscale/dn_gscale NVFP4: fp32 [num_experts] each; MX: NULL
 *   expert_ids int32 [tokens][topk]; weights fp32 [tokens][topk]
 *   x        bf16 [tokens][hidden]
 *   h        workspace of tokens*topk*dff*10 bytes (caller-owned, 16-byte
 *            aligned): fp32 h [tokens][topk][2*dff], then bf16 a
 *            [tokens][topk][dff]; both are left holding the call's values
 *   y        fp32 [tokens][hidden]
 *   hidden, dff multiples of the block size (32 MX, 16 NVFP4); tokens 1 .. MXQ_MAX_BATCH;
 *   topk 1 .. MXQ_MAX_TOPK with topk rounded up to a power of two, times 2*dff
 *   bytes, at most 64 KiB (else MXQ_E_UNSUPPORTED)
 */
mxq_status_t mxq_moe_block(mxq_format_t fmt, const uint8_t *gu_codes, const uint8_t *gu_scales, const float *gu_gscale,
                           const uint8_t *dn_codes, const uint8_t *dn_scales, const float *dn_gscale,
                           const int32_t *expert_ids, const float *weights, const uint16_t *x, float *h, float *y,
                           int64_t num_experts, int64_t hidden, int64_t dff, int64_t tokens, int64_t topk,
                           void *stream);

/*
 * MoE decode block with the routing of mxq_moe_route done in place: the
 * gate/up kernel selects each token's experts and weights from its router
 * logits (the same selection and the same fp32 weights, bit for bit, as
 * mxq_moe_route), writes them to expert_ids and weights, and the block then
 * proceeds as mxq_moe_block.  One launch fewer than mxq_moe_route followed by
 * mxq_moe_block.
 *   logits      fp32 [tokens][num_experts], num_experts 1 .. 1024, no NaN
 *   renorm      nonzero: weights divided by the sum of the selected ones
 *   expert_ids  int32 [tokens][topk] out;  weights fp32 [tokens][topk] out
 *   topk        at most num_experts (else MXQ_E_SHAPE)
 * Every other argument, limit and error as mxq_moe_block.
 */
mxq_status_t mxq_moe_block_routed(mxq_format_t fmt, const uint8_t *gu_codes, const uint8_t *gu_scales,
                                  const float *gu_gscale, const uint8_t *dn_codes, const uint8_t *dn_scales,
                                  const float *dn_gscale, const float *logits, int renorm, int32_t *expert_ids,
                                  float *weights, const uint16_t *x, float *h, float *y, int64_t num_experts,
                                  int64_t hidden, int64_t dff, int64_t tokens, int64_t topk, void *stream);

/*
 * Allocation-free MoE decode block, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and arguments as
 * mxq_moe_block without `h`; the workspace (h and a) goes to a static device
 * array of 2.5 MiB that the library holds on each GPU it runs on until the
 * process ends (looked up once per device; the call allocates nothing).
 *   tokens * topk * dff * 10 bytes at most 2.5 MiB (every call the LDS limit
 *   above admits fits), else MXQ_E_UNSUPPORTED; MXQ_E_DEVICE if the array's
 *   address cannot be obtained.
 * All calls on one GPU share the array: calls that overlap in time on one GPU
 * (different streams, or several host threads) race and must be serialised
 * by the caller.  The array needs no clearing (each call writes the parts it
 * reads before reading them).
 */
mxq_status_t mxq_moe_block_noalloc(mxq_format_t fmt, const uint8_t *gu_codes, const uint8_t *gu_scales,
                                   const float *gu_gscale, const uint8_t *dn_codes, const uint8_t *dn_scales,
                                   const float *dn_gscale, const int32_t *expert_ids, const float *weights,
                                   const uint16_t *x, float *y, int64_t num_experts, int64_t hidden, int64_t dff,
                                   int64_t tokens, int64_t topk, void *stream);

/*
 * Expert-batched MoE GEMM (prefill).  The "Decoding block-float formats in
 * software" section of the "MLxcel 0.8 release" post credits a kernel that
 * processes the tokens expert by expert for its MXFP4 MoE prefill gain; here
 * each expert's weights are decoded to bf16 and multiplied on the matrix unit
 * with the inputs of the (token, slot) pairs routed to it (fp32 accumulate):
 * one kernel streams each expert's rows against 64 of its pairs at a time,
 * finding them in the ids itself (no host sync, no grouping pass), in every
 * format and at every k:
 *
 *   y[t][s][i] = sum_k W[expert_ids[t][s]][i][k] * x_ts[k]
 *   x_ts = x[t] (x_per_slot == 0, e.g. gate/up) or x[t][s] (x_per_slot != 0, e.g. down)
 *
 *   codes/scales   bank [num_experts][n][...] (layout as mxq_moe_gemv)
 *   global_scale   NVFP4: fp32 [num_experts]; MX: NULL
 *   expert_ids     int32 [m][topk]; x bf16 [m][k] or [m][topk][k]
 *   y              [m][topk][n], bf16 (RNE of the fp32 value) or fp32 (y_dtype)
 *   workspace      int32 [num_experts + 1 + m * topk], caller-owned, 4-byte
 *                  aligned scratch; the current kernel neither reads nor
 *                  writes it
 *   m 1 .. 2^24 / topk;  topk 1 .. MXQ_MAX_TOPK;  num_experts 1 .. 1024;
 *   n >= 1;  k a positive multiple of the block size (32 MX, 16 NVFP4), up
 *   to 2^31 - 1
 * A pair whose id is outside [0, num_experts) gets a NaN output row.  The
 * kernel runs on `stream`.
 */
mxq_status_t mxq_moe_gemm(mxq_format_t fmt, const uint8_t *codes, const uint8_t *scales, const float *global_scale,
                          const int32_t *expert_ids, const uint16_t *x, int x_per_slot, void *y, mxq_out_t y_dtype,
                          int32_t *workspace, int64_t num_experts, int64_t m, int64_t n, int64_t k, int64_t topk,
                          void *stream);

/*
 * Block-float quantizer: bf16 values -> packed codes and block scales, the
 * layout every other entry point reads.  The ROCm status table of the "Build
 * from source" manual (section "Current status", row "mxfp8, mxfp4
 * checkpoints") requantizes vendor FP8 block checkpoints to MXFP8 at load;
 * the pages give no procedure, so the conversion is the OCP MX v1.0 one:
 *   MX:    per 32-element block, X = 2^(floor(log2 max|v|) - emax) with emax 2
 *          (E2M1) or 8 (E4M3), the exponent clamped to [-127, 127] (a zero
 *          block takes -127) and stored as the E8M0 byte; codes = q(v / X).
 *   NVFP4: per 16-element block, s = E4M3 rounding of fl32(max|v| / fl32(6 g))
 *          for the caller's per-tensor scale g = global_scale[0] > 0;
 *          codes = q(fl32(v / fl32(s g))), or +-0 when s is 0.
 *   q(p):  the sign of p and |p| rounded to the nearest value of the element
 *          format, ties to the even code, saturating at its largest value.
 *   x       bf16 [rows][k], 16-byte aligned, finite values
 *   codes   out [rows][k/2] (E2M1, low nibble = even k) or [rows][k] (E4M3), 16-byte aligned
 *   scales  out [rows][k/32] (E8M0) or [rows][k/16] (E4M3)
 *   global_scale  NVFP4: device fp32 [1], input; MX: NULL
 *   k a positive multiple of the block size; rows * k <= 2^36
 */
mxq_status_t mxq_quantize(mxq_format_t fmt, const uint16_t *x, const float *global_scale, uint8_t *codes, uint8_t *scales,
                          int64_t rows, int64_t k, void *stream);

/*
 * FP8 block checkpoint -> MXFP8.  The ROCm status table of the "Build from
 * source" manual (section "Current status", row "mxfp8, mxfp4 checkpoints")
 * converts vendor FP8 checkpoints to MXFP8 when a model loads; such a
 * checkpoint stores E4M3 codes with one fp32 scale per 128 x 128 tile.  The
 * pages give no procedure; the conversion dequantizes and requantizes:
 *   v = fl32(E4M3(c) * s)   s = tile_scales[r / block_n][j / block_k]
 *   then, per 32-element block of a row, the OCP MX conversion of mxq_quantize
 *   (shared exponent floor(log2 max|v|) - 8, clamped to [-127, 127]; codes =
 *   the nearest E4M3 values of v / 2^exponent, ties to the even code,
 *   saturating at 448, sign kept).
 *   codes_in     E4M3 [n][k], 16-byte aligned; finite values (no 0x7F / 0xFF)
 *   tile_scales  fp32 [ceil(n / block_n)][ceil(k / block_k)], row-major; the
 *                products E4M3 * scale must be finite fp32 numbers
 *   codes        out E4M3 [n][k], 16-byte aligned (may not alias codes_in)
 *   scales       out E8M0 [n][k / 32]
 *   k and block_k multiples of 32 (a block never straddles two tiles);
 *   n * k <= 2^36.  Results for non-finite inputs are unspecified.
 */
mxq_status_t mxq_requant_fp8(const uint8_t *codes_in, const float *tile_scales, uint8_t *codes, uint8_t *scales,
                             int64_t n, int64_t k, int64_t block_n, int64_t block_k, void *stream);

/*
 * Measurement reference: a plain streaming read of `bytes` bytes at `data`
 * (16-byte loads with the nontemporal hint, as the GEMV reads its codes, on 8
 * workgroups per compute unit), the achievable bandwidth the GEMV kernels are
 * compared with ("The memory wall" section of the post, slide 15 of the talk:
 * decode time is the time to stream the weights).  layout 0: lanes
 * interleaved over the range; 1: one contiguous range per workgroup (other
 * values: MXQ_E_FORMAT).  The words read are XOR-folded into
 * sink[0 .. workgroups), so the loads cannot be dropped.
 *   data        16-byte aligned;  bytes a positive multiple of 16
 *   sink        uint32 [sink_words]; sink_words >= 8 * compute units (256 CUs:
 *               2048), else MXQ_E_UNSUPPORTED
 */
mxq_status_t mxq_stream_read(const void *data, int64_t bytes, int layout, uint32_t *sink, int64_t sink_words,
                             void *stream);

/* Static description of a status code (never NULL). */
const char *mxq_status_string(int status);

/* ABI version of this header: 9 (mxq_moe_block_routed added to 8). */
int mxq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
