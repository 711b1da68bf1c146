"""Python binding of libmxq: block-float (MXFP4 / MXFP8 / NVFP4) quantized GEMV,
expert-indexed MoE GEMV and prefill GEMM on AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmxq.so`` behind the C ABI in ``include/mxq.h``.  PyTorch
supplies device memory and the current stream.  There is no fallback: if the
library is missing or the device is not gfx950 the calls raise.

Tensors:
  codes   uint8, [n, k/2] (E2M1) or [n, k] (E4M3); MoE banks [E, n, ...]
  scales  uint8, [n, k/32] (E8M0) or [n, k/16] (E4M3 for NVFP4)
  x       bfloat16, [batch, k] (or [tokens, topk, k] for per-slot MoE input)
  global_scale  float32 [1] (dense NVFP4) or [E] (MoE NVFP4), None for MX
"""
from __future__ import annotations

import ctypes
import os

import torch

MXFP4, MXFP8, NVFP4 = 1, 2, 3
FORMATS = {"mxfp4": MXFP4, "mxfp8": MXFP8, "nvfp4": NVFP4}
BLOCK = {MXFP4: 32, MXFP8: 32, NVFP4: 16}
OUT_F32, OUT_BF16 = 0, 1
STATUS = {0: "MXQ_OK", 1: "MXQ_E_NULLPTR", 2: "MXQ_E_SHAPE", 3: "MXQ_E_ALIGN", 4: "MXQ_E_FORMAT",
          5: "MXQ_E_UNSUPPORTED", 6: "MXQ_E_DEVICE", 7: "MXQ_E_LAUNCH"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxq.so")


class MxqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


class GemvConfig(ctypes.Structure):
    """mxq_gemv_config_t: the dense GEMV's kernel and tile, for tests and tuning (0 = chosen from the shape)."""
    _fields_ = [(f, ctypes.c_int32) for f in ("path", "rows_g", "rows_s", "rows_r", "mm_r", "mm_s", "mfma_r",
                                               "mfma_ks", "mfma_nw", "per_cu", "grid")]


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mxq_gemv.argtypes = [I, P, P, P, P, P, I64, I64, I64, P]
        L.mxq_gemv_config.argtypes = [I, P, P, P, P, P, I64, I64, I64, ctypes.POINTER(GemvConfig), P]
        L.mxq_moe_gemv.argtypes = [I, P, P, P, P, P, I, P, I64, I64, I64, I64, I64, P]
        L.mxq_gemm.argtypes = [I, P, P, P, P, P, I, I64, I64, I64, P]
        L.mxq_dequant.argtypes = [I, P, P, P, P, I64, I64, P]
        L.mxq_moe_route.argtypes = [P, P, P, I64, I64, I64, I, P]
        L.mxq_moe_block.argtypes = [I, P, P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P]
        L.mxq_moe_block_noalloc.argtypes = [I, P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P]
        L.mxq_moe_block_routed.argtypes = [I, P, P, P, P, P, P, P, I, P, P, P, P, P, I64, I64, I64, I64, I64, P]
        L.mxq_moe_gemm.argtypes = [I, P, P, P, P, P, I, P, I, P, I64, I64, I64, I64, I64, P]
        L.mxq_quantize.argtypes = [I, P, P, P, P, I64, I64, P]
        L.mxq_requant_fp8.argtypes = [P, P, P, P, I64, I64, I64, I64, P]
        L.mxq_stream_read.argtypes = [P, I64, I, P, I64, P]
        for f in (L.mxq_gemv, L.mxq_gemv_config, L.mxq_moe_gemv, L.mxq_gemm, L.mxq_dequant, L.mxq_moe_route, L.mxq_moe_block,
                  L.mxq_moe_block_noalloc, L.mxq_moe_block_routed, L.mxq_moe_gemm, L.mxq_quantize, L.mxq_requant_fp8, L.mxq_stream_read):
            f.restype = I
        L.mxq_status_string.argtypes = [I]
        L.mxq_status_string.restype = ctypes.c_char_p
        L.mxq_abi_version.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mxq_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _check(st, what):
    if st != 0:
        raise MxqError(st, what)


def _k_of(fmt, codes):
    return codes.shape[-1] if fmt == MXFP8 else 2 * codes.shape[-1]


def _check_weight(fmt, codes, scales, global_scale, experts=None):
    """Host-side shape checks: the C ABI takes raw pointers and cannot see sizes."""
    if fmt not in BLOCK:
        raise ValueError(f"unknown format {fmt}")
    lead = 2 if experts is not None else 1
    if codes.dim() != lead + 1 or scales.dim() != lead + 1:
        raise ValueError(f"codes and scales must have {lead + 1} dimensions")
    k = _k_of(fmt, codes)
    if k % BLOCK[fmt]:
        raise ValueError(f"k={k} is not a multiple of the block size {BLOCK[fmt]}")
    if tuple(scales.shape) != tuple(codes.shape[:-1]) + (k // BLOCK[fmt],):
        raise ValueError(f"scales shape {tuple(scales.shape)} does not match codes {tuple(codes.shape)}")
    if (global_scale is None) != (fmt != NVFP4):
        raise ValueError("NVFP4 needs global_scale; MX formats take none")
    if global_scale is not None and global_scale.numel() < (experts if experts is not None else 1):
        raise ValueError("global_scale has too few elements")
    return k


def gemv(fmt, codes, scales, x, global_scale=None, out=None, stream=None, config=None):
    """y[b][i] = sum_k W[i][k] * x[b][k] -> float32 [batch, n].  config: a dict of mxq_gemv_config_t
    fields (the kernel and tile chosen by the caller, through mxq_gemv_config), None for mxq_gemv."""
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    x = _dev(x, torch.bfloat16, "x")
    global_scale = _dev(global_scale, torch.float32, "global_scale")
    k = _check_weight(fmt, codes, scales, global_scale)
    n = codes.shape[0]
    x2 = x.reshape(-1, x.shape[-1])
    if x2.shape[1] != k:
        raise ValueError(f"x has k={x2.shape[1]}, weights have k={k}")
    batch = x2.shape[0]
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=codes.device)
    out = _dev(out, torch.float32, "out")
    if out.numel() != batch * n:
        raise ValueError("out must hold batch * n elements")
    if config is not None:
        cfg = GemvConfig(**config)
        _check(lib().mxq_gemv_config(fmt, _ptr(codes), _ptr(scales), _ptr(global_scale), _ptr(x2), _ptr(out), n, k,
                                     batch, ctypes.byref(cfg), _stream(stream)), "mxq_gemv_config")
        return out
    _check(lib().mxq_gemv(fmt, _ptr(codes), _ptr(scales), _ptr(global_scale), _ptr(x2), _ptr(out), n, k, batch,
                          _stream(stream)), "mxq_gemv")
    return out


def moe_gemv(fmt, codes, scales, expert_ids, x, x_per_slot, global_scale=None, out=None, stream=None):
    """y[t][s][i] = sum_k W[ids[t][s]][i][k] * x_ts[k] -> float32 [tokens, topk, n]."""
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    expert_ids = _dev(expert_ids, torch.int32, "expert_ids")
    x = _dev(x, torch.bfloat16, "x")
    global_scale = _dev(global_scale, torch.float32, "global_scale")
    experts, n = codes.shape[0], codes.shape[1]
    k = _check_weight(fmt, codes, scales, global_scale, experts=experts)
    if expert_ids.dim() != 2:
        raise ValueError("expert_ids must be [tokens, topk]")
    tokens, topk = expert_ids.shape
    want = (tokens, topk, k) if x_per_slot else (tokens, k)
    if tuple(x.shape) != want:
        raise ValueError(f"x must have shape {want}, got {tuple(x.shape)}")
    if out is None:
        out = torch.empty((tokens, topk, n), dtype=torch.float32, device=codes.device)
    out = _dev(out, torch.float32, "out")
    if out.numel() != tokens * topk * n:
        raise ValueError("out must hold tokens * topk * n elements")
    _check(lib().mxq_moe_gemv(fmt, _ptr(codes), _ptr(scales), _ptr(global_scale), _ptr(expert_ids), _ptr(x),
                              1 if x_per_slot else 0, _ptr(out), experts, n, k, tokens, topk, _stream(stream)),
           "mxq_moe_gemv")
    return out


def moe_route(logits, topk, renorm=False, ids=None, weights=None, stream=None):
    """Top-k softmax routing of float32 logits [tokens, experts] -> (int32 ids, float32 weights), [tokens, topk]."""
    logits = _dev(logits, torch.float32, "logits")
    if logits.dim() != 2:
        raise ValueError("logits must be [tokens, experts]")
    tokens, experts = logits.shape
    if ids is None:
        ids = torch.empty((tokens, topk), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((tokens, topk), dtype=torch.float32, device=logits.device)
    ids = _dev(ids, torch.int32, "ids")
    weights = _dev(weights, torch.float32, "weights")
    if ids.numel() != tokens * topk or weights.numel() != tokens * topk:
        raise ValueError("ids and weights must hold tokens * topk elements")
    _check(lib().mxq_moe_route(_ptr(logits), _ptr(ids), _ptr(weights), tokens, experts, topk, 1 if renorm else 0,
                               _stream(stream)), "mxq_moe_route")
    return ids, weights


def moe_block_workspace_elems(tokens, topk, dff):
    """float32 elements of the MoE block's workspace: tokens * topk * dff * 10 bytes."""
    return tokens * topk * dff * 10 // 4


def moe_block_workspace_views(h, tokens, topk, dff):
    """(gate/up outputs float32 [tokens, topk, 2 dff], activations bfloat16 [tokens, topk, dff]) of a workspace."""
    flat = h.reshape(-1)
    n = tokens * topk * 2 * dff
    act = flat[n:n + tokens * topk * dff // 2].view(torch.bfloat16)
    return flat[:n].view(tokens, topk, 2 * dff), act.view(tokens, topk, dff)


def moe_block(fmt, gu_codes, gu_scales, dn_codes, dn_scales, expert_ids, weights, x, gu_global_scale=None,
              dn_global_scale=None, h=None, out=None, stream=None, noalloc=False):
    """MoE decode block -> float32 [tokens, hidden]: y[t] = sum_s w[t][s] * W_dn[e] . bf16(silu(gate) * up),
    with gate/up = W_gu[e] . x[t] (rows [0, dff) and [dff, 2 dff) of the gate/up bank).
    h is the workspace (allocated when None): moe_block_workspace_elems(tokens, topk, dff) float32
    elements holding the float32 gate/up outputs [tokens, topk, 2 dff], then the bfloat16 activations
    [tokens, topk, dff] (see moe_block_workspace_views).  With noalloc the call goes to
    mxq_moe_block_noalloc, whose workspace is the library's static device array (h must be None; `out`
    is still allocated here when None)."""
    gu_codes = _dev(gu_codes, torch.uint8, "gu_codes")
    gu_scales = _dev(gu_scales, torch.uint8, "gu_scales")
    dn_codes = _dev(dn_codes, torch.uint8, "dn_codes")
    dn_scales = _dev(dn_scales, torch.uint8, "dn_scales")
    expert_ids = _dev(expert_ids, torch.int32, "expert_ids")
    weights = _dev(weights, torch.float32, "weights")
    x = _dev(x, torch.bfloat16, "x")
    gu_global_scale = _dev(gu_global_scale, torch.float32, "gu_global_scale")
    dn_global_scale = _dev(dn_global_scale, torch.float32, "dn_global_scale")
    experts, two_dff = gu_codes.shape[0], gu_codes.shape[1]
    hidden = _check_weight(fmt, gu_codes, gu_scales, gu_global_scale, experts=experts)
    dff = _check_weight(fmt, dn_codes, dn_scales, dn_global_scale, experts=experts)
    if two_dff != 2 * dff or tuple(dn_codes.shape[:2]) != (experts, hidden):
        raise ValueError(f"gate/up bank {tuple(gu_codes.shape)} and down bank {tuple(dn_codes.shape)} disagree")
    if expert_ids.dim() != 2 or tuple(weights.shape) != tuple(expert_ids.shape):
        raise ValueError("expert_ids and weights must both be [tokens, topk]")
    tokens, topk = expert_ids.shape
    if tuple(x.shape) != (tokens, hidden):
        raise ValueError(f"x must have shape {(tokens, hidden)}, got {tuple(x.shape)}")
    if noalloc:
        if h is not None:
            raise ValueError("noalloc takes no workspace")
    else:
        need = moe_block_workspace_elems(tokens, topk, dff)
        if h is None:
            h = torch.empty(need, dtype=torch.float32, device=gu_codes.device)
        h = _dev(h, torch.float32, "h")
        if h.numel() < need:
            raise ValueError(f"h must hold moe_block_workspace_elems(tokens, topk, dff) = {need} elements")
    if out is None:
        out = torch.empty((tokens, hidden), dtype=torch.float32, device=gu_codes.device)
    out = _dev(out, torch.float32, "out")
    if out.numel() != tokens * hidden:
        raise ValueError("out must hold tokens * hidden elements")
    if noalloc:
        _check(lib().mxq_moe_block_noalloc(fmt, _ptr(gu_codes), _ptr(gu_scales), _ptr(gu_global_scale),
                                           _ptr(dn_codes), _ptr(dn_scales), _ptr(dn_global_scale), _ptr(expert_ids),
                                           _ptr(weights), _ptr(x), _ptr(out), experts, hidden, dff, tokens, topk,
                                           _stream(stream)),
               "mxq_moe_block_noalloc")
        return out
    _check(lib().mxq_moe_block(fmt, _ptr(gu_codes), _ptr(gu_scales), _ptr(gu_global_scale), _ptr(dn_codes),
                               _ptr(dn_scales), _ptr(dn_global_scale), _ptr(expert_ids), _ptr(weights), _ptr(x),
                               _ptr(h), _ptr(out), experts, hidden, dff, tokens, topk, _stream(stream)),
           "mxq_moe_block")
    return out


def moe_block_routed(fmt, gu_codes, gu_scales, dn_codes, dn_scales, logits, topk, x, renorm=False,
                     gu_global_scale=None, dn_global_scale=None, h=None, out=None, ids=None, weights=None,
                     stream=None):
    """MoE decode block that routes in place from float32 router logits [tokens, experts] (the selection
    and weights of moe_route, bit for bit) -> (float32 y [tokens, hidden], int32 ids [tokens, topk],
    float32 weights [tokens, topk]).  h as in moe_block (allocated when None)."""
    gu_codes = _dev(gu_codes, torch.uint8, "gu_codes")
    gu_scales = _dev(gu_scales, torch.uint8, "gu_scales")
    dn_codes = _dev(dn_codes, torch.uint8, "dn_codes")
    dn_scales = _dev(dn_scales, torch.uint8, "dn_scales")
    logits = _dev(logits, torch.float32, "logits")
    x = _dev(x, torch.bfloat16, "x")
    gu_global_scale = _dev(gu_global_scale, torch.float32, "gu_global_scale")
    dn_global_scale = _dev(dn_global_scale, torch.float32, "dn_global_scale")
    experts, two_dff = gu_codes.shape[0], gu_codes.shape[1]
    hidden = _check_weight(fmt, gu_codes, gu_scales, gu_global_scale, experts=experts)
    dff = _check_weight(fmt, dn_codes, dn_scales, dn_global_scale, experts=experts)
    if two_dff != 2 * dff or tuple(dn_codes.shape[:2]) != (experts, hidden):
        raise ValueError(f"gate/up bank {tuple(gu_codes.shape)} and down bank {tuple(dn_codes.shape)} disagree")
    if logits.dim() != 2 or logits.shape[1] != experts:
        raise ValueError(f"logits must be [tokens, {experts}], got {tuple(logits.shape)}")
    tokens = logits.shape[0]
    if tuple(x.shape) != (tokens, hidden):
        raise ValueError(f"x must have shape {(tokens, hidden)}, got {tuple(x.shape)}")
    dev = gu_codes.device
    need = moe_block_workspace_elems(tokens, topk, dff)
    if h is None:
        h = torch.empty(need, dtype=torch.float32, device=dev)
    h = _dev(h, torch.float32, "h")
    if h.numel() < need:
        raise ValueError(f"h must hold moe_block_workspace_elems(tokens, topk, dff) = {need} elements")
    if out is None:
        out = torch.empty((tokens, hidden), dtype=torch.float32, device=dev)
    if ids is None:
        ids = torch.empty((tokens, topk), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((tokens, topk), dtype=torch.float32, device=dev)
    out = _dev(out, torch.float32, "out")
    ids = _dev(ids, torch.int32, "ids")
    weights = _dev(weights, torch.float32, "weights")
    if out.numel() != tokens * hidden:
        raise ValueError("out must hold tokens * hidden elements")
    if ids.numel() != tokens * topk or weights.numel() != tokens * topk:
        raise ValueError("ids and weights must hold tokens * topk elements")
    _check(lib().mxq_moe_block_routed(fmt, _ptr(gu_codes), _ptr(gu_scales), _ptr(gu_global_scale),
                                      _ptr(dn_codes), _ptr(dn_scales), _ptr(dn_global_scale), _ptr(logits),
                                      1 if renorm else 0, _ptr(ids), _ptr(weights), _ptr(x), _ptr(h), _ptr(out),
                                      experts, hidden, dff, tokens, topk, _stream(stream)),
           "mxq_moe_block_routed")
    return out, ids, weights


def gemm(fmt, codes, scales, x, global_scale=None, out_dtype=torch.bfloat16, out=None, stream=None):
    """Y[m][i] = sum_k X[m][k] * W[i][k] -> [m, n] in float32 or bfloat16 (RNE)."""
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    x = _dev(x, torch.bfloat16, "x")
    global_scale = _dev(global_scale, torch.float32, "global_scale")
    k = _check_weight(fmt, codes, scales, global_scale)
    n = codes.shape[0]
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}], got {tuple(x.shape)}")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=codes.device)
    out = _dev(out, out_dtype, "out")
    if out.numel() != m * n:
        raise ValueError("out must hold m * n elements")
    ydt = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    _check(lib().mxq_gemm(fmt, _ptr(codes), _ptr(scales), _ptr(global_scale), _ptr(x), _ptr(out), ydt, m, n, k,
                          _stream(stream)), "mxq_gemm")
    return out


def moe_gemm(fmt, codes, scales, expert_ids, x, x_per_slot=0, global_scale=None, out_dtype=torch.bfloat16, out=None,
             workspace=None, stream=None):
    """Expert-batched MoE GEMM: y[t][s][i] = sum_k W[ids[t][s]][i][k] * x_ts[k] -> [m, topk, n] in float32 or
    bfloat16 (RNE); x_ts = x[t] ([m, k]) or x[t][s] ([m, topk, k], x_per_slot).  workspace: int32
    [experts + 1 + m * topk] (allocated when None)."""
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    expert_ids = _dev(expert_ids, torch.int32, "expert_ids")
    x = _dev(x, torch.bfloat16, "x")
    global_scale = _dev(global_scale, torch.float32, "global_scale")
    experts, n = codes.shape[0], codes.shape[1]
    k = _check_weight(fmt, codes, scales, global_scale, experts=experts)
    if expert_ids.dim() != 2:
        raise ValueError("expert_ids must be [m, topk]")
    m, topk = expert_ids.shape
    want = (m, topk, k) if x_per_slot else (m, k)
    if tuple(x.shape) != want:
        raise ValueError(f"x must have shape {want}, got {tuple(x.shape)}")
    if out is None:
        out = torch.empty((m, topk, n), dtype=out_dtype, device=codes.device)
    out = _dev(out, out_dtype, "out")
    if out.numel() != m * topk * n:
        raise ValueError("out must hold m * topk * n elements")
    if workspace is None:
        workspace = torch.empty((experts + 1 + m * topk,), dtype=torch.int32, device=codes.device)
    workspace = _dev(workspace, torch.int32, "workspace")
    if workspace.numel() < experts + 1 + m * topk:
        raise ValueError("workspace must hold experts + 1 + m * topk int32")
    ydt = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    _check(lib().mxq_moe_gemm(fmt, _ptr(codes), _ptr(scales), _ptr(global_scale), _ptr(expert_ids), _ptr(x),
                              1 if x_per_slot else 0, _ptr(out), ydt, _ptr(workspace), experts, m, n, k, topk,
                              _stream(stream)),
           "mxq_moe_gemm")
    return out


def quantize(fmt, x, global_scale=None, codes=None, scales=None, stream=None):
    """bf16 x [rows, k] -> (codes uint8 [rows, k/2] or [rows, k], scales uint8 [rows, k/block]); NVFP4 takes its
    per-tensor scale as a float32 [1] device tensor."""
    x = _dev(x, torch.bfloat16, "x")
    global_scale = _dev(global_scale, torch.float32, "global_scale")
    if x.dim() != 2:
        raise ValueError("x must be [rows, k]")
    rows, k = x.shape
    cb = k if fmt == MXFP8 else k // 2
    if codes is None:
        codes = torch.empty((rows, cb), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, k // BLOCK.get(fmt, 32)), dtype=torch.uint8, device=x.device)
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    if codes.numel() != rows * cb or scales.numel() != rows * (k // BLOCK.get(fmt, 32)):
        raise ValueError("codes / scales do not match x")
    _check(lib().mxq_quantize(fmt, _ptr(x), _ptr(global_scale), _ptr(codes), _ptr(scales), rows, k,
                              _stream(stream)), "mxq_quantize")
    return codes, scales


def requant_fp8(codes_in, tile_scales, block_n=128, block_k=128, codes=None, scales=None, stream=None):
    """FP8 block checkpoint -> MXFP8: E4M3 codes uint8 [n, k] with float32 tile scales
    [ceil(n / block_n), ceil(k / block_k)] -> (codes uint8 [n, k], E8M0 scales uint8 [n, k / 32])."""
    codes_in = _dev(codes_in, torch.uint8, "codes_in")
    tile_scales = _dev(tile_scales, torch.float32, "tile_scales")
    if codes_in.dim() != 2:
        raise ValueError("codes_in must be [n, k]")
    n, k = codes_in.shape
    want = ((n + block_n - 1) // block_n, (k + block_k - 1) // block_k)
    if tuple(tile_scales.shape) != want:
        raise ValueError(f"tile_scales must have shape {want}, got {tuple(tile_scales.shape)}")
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.uint8, device=codes_in.device)
    if scales is None:
        scales = torch.empty((n, k // 32), dtype=torch.uint8, device=codes_in.device)
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    if codes.numel() != n * k or scales.numel() != n * (k // 32):
        raise ValueError("codes / scales do not match codes_in")
    _check(lib().mxq_requant_fp8(_ptr(codes_in), _ptr(tile_scales), _ptr(codes), _ptr(scales), n, k, block_n, block_k,
                                 _stream(stream)), "mxq_requant_fp8")
    return codes, scales


def dequant(fmt, codes, scales, global_scale=None, out=None, stream=None):
    """Decoded fp32 weights [rows, k] (same device decode as the other kernels)."""
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    global_scale = _dev(global_scale, torch.float32, "global_scale")
    k = _check_weight(fmt, codes, scales, global_scale)
    rows = codes.shape[0]
    if out is None:
        out = torch.empty((rows, k), dtype=torch.float32, device=codes.device)
    out = _dev(out, torch.float32, "out")
    if out.numel() != rows * k:
        raise ValueError("out must hold rows * k elements")
    _check(lib().mxq_dequant(fmt, _ptr(codes), _ptr(scales), _ptr(global_scale), _ptr(out), rows, k,
                             _stream(stream)), "mxq_dequant")
    return out


def stream_read(data, sink, nbytes=None, layout=0, stream=None):
    """Streaming read of the first nbytes (default: all) of a contiguous device tensor (the
    achievable-bandwidth reference; layout 0 interleaved, 1 contiguous range per workgroup);
    sink: int32 device tensor of at least 8 words per CU."""
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous device tensor")
    sink = _dev(sink, torch.int32, "sink")
    nb = data.numel() * data.element_size() if nbytes is None else int(nbytes)
    if nb > data.numel() * data.element_size():
        raise ValueError("nbytes exceeds the tensor")
    _check(lib().mxq_stream_read(_ptr(data), nb, int(layout), _ptr(sink), sink.numel(), _stream(stream)),
           "mxq_stream_read")


def weight_bytes(fmt, n, k):
    """Algorithmic bytes of one weight matrix: codes + block scales (+4 for NVFP4's fp32 scale)."""
    codes = n * k if fmt == MXFP8 else n * k // 2
    return codes + n * (k // BLOCK[fmt]) + (4 if fmt == NVFP4 else 0)
