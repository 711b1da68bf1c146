"""CPU oracle for the block-float quantized GEMV / MoE GEMV / prefill GEMM.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It is a plain C
library (``oracle.c``, built with gcc -O2, OpenMP over output rows, no
-ffast-math) behind numpy-facing ctypes wrappers.  It shares no code with the
HIP library.

Every function returns fp64 results; the GEMV-style ones also return
``abs_y = sum_k |w*x|`` so a test can apply the acceptance bound
``|y_gpu - y| <= 1e-5 * abs_y + 1e-6``.

Pins (tests/test_oracle_*.py): E2M1 value table, E8M0 closed form and
``torch.float8_e8m0fnu``, E4M3 against ``torch.float8_e4m3fn``, the
scale-bump invariant, exact rational brute force on 4x32 inputs (dense, MoE and
GEMM rows), one-hot activations and closed-form sums.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MXFP4, MXFP8, NVFP4 = 1, 2, 3
BLOCK = {MXFP4: 32, MXFP8: 32, NVFP4: 16}


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for name in ("orc_e2m1", "orc_e8m0", "orc_e4m3"):
            getattr(lib, name).restype = ctypes.c_double
            getattr(lib, name).argtypes = [ctypes.c_uint]
        lib.orc_bf16.restype = ctypes.c_double
        lib.orc_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_num_threads.restype = I
        lib.orc_set_num_threads.argtypes = [I]
        lib.orc_dequant.argtypes = [I, P, P, P, I64, I64, P]
        lib.orc_gemv.argtypes = [I, P, P, P, P, I64, I64, I64, P, P]
        lib.orc_moe_gemv.argtypes = [I, P, P, P, P, P, I, I64, I64, I64, I64, I64, P, P]
        lib.orc_gemm_rows.argtypes = [I, P, P, P, P, P, I64, I64, I64, P, P]
        lib.orc_moe_route.argtypes = [P, I64, I64, I64, I, P, P]
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_round_bf16.argtypes = [ctypes.c_double]
        lib.orc_round_bf16.restype = ctypes.c_double
        D = ctypes.c_double
        lib.orc_moe_block.argtypes = [I, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, D, D, D, P, P, P]
        lib.orc_quantize.argtypes = [I, P, ctypes.c_float, I64, I64, P, P]
        lib.orc_requant_fp8.argtypes = [P, P, I64, I64, I64, I64, P, P]
        lib.orc_split_e4m3.argtypes = [P, I64, I64, P, P, P, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _check(fmt, k):
    if fmt not in BLOCK:
        raise ValueError(f"unknown format {fmt}")
    if k % BLOCK[fmt]:
        raise ValueError(f"k={k} is not a multiple of the block size {BLOCK[fmt]}")


def e2m1(c: int) -> float:
    return _load().orc_e2m1(c)


def e8m0(u: int) -> float:
    return _load().orc_e8m0(u)


def e4m3(b: int) -> float:
    return _load().orc_e4m3(b)


def bf16(h: int) -> float:
    return _load().orc_bf16(h)


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(n)


def dequant(fmt, codes, scales, g, rows, k):
    """fp32 [rows][k] decoded weights."""
    _check(fmt, k)
    codes, scales, g = _c(codes, np.uint8), _c(scales, np.uint8), _c(g, np.float32)
    w = np.empty((rows, k), dtype=np.float32)
    _load().orc_dequant(fmt, _ptr(codes), _ptr(scales), _ptr(g), rows, k, _ptr(w))
    return w


def gemv(fmt, codes, scales, g, x, n, k):
    """(y, abs_y), both fp64 [batch][n]; x is bf16 bits uint16 [batch][k]."""
    _check(fmt, k)
    codes, scales, g = _c(codes, np.uint8), _c(scales, np.uint8), _c(g, np.float32)
    x = _c(x, np.uint16).reshape(-1, k)
    batch = x.shape[0]
    y = np.empty((batch, n), dtype=np.float64)
    a = np.empty((batch, n), dtype=np.float64)
    _load().orc_gemv(fmt, _ptr(codes), _ptr(scales), _ptr(g), _ptr(x), batch, n, k, _ptr(y), _ptr(a))
    return y, a


def moe_gemv(fmt, codes, scales, g, ids, x, x_per_slot, experts, n, k):
    """(y, abs_y), both fp64 [tokens][topk][n]."""
    _check(fmt, k)
    codes, scales, g = _c(codes, np.uint8), _c(scales, np.uint8), _c(g, np.float32)
    ids = _c(ids, np.int32)
    tokens, topk = ids.shape
    x = _c(x, np.uint16)
    y = np.empty((tokens, topk, n), dtype=np.float64)
    a = np.empty((tokens, topk, n), dtype=np.float64)
    _load().orc_moe_gemv(fmt, _ptr(codes), _ptr(scales), _ptr(g), _ptr(ids), _ptr(x), int(x_per_slot),
                         experts, n, k, tokens, topk, _ptr(y), _ptr(a))
    return y, a


def gemm_rows(fmt, codes, scales, g, X, rows, n, k):
    """(Y, abs_Y), both fp64 [len(rows)][n], for the listed token rows of X [m][k]."""
    _check(fmt, k)
    codes, scales, g = _c(codes, np.uint8), _c(scales, np.uint8), _c(g, np.float32)
    X = _c(X, np.uint16)
    rows = _c(rows, np.int64)
    Y = np.empty((rows.size, n), dtype=np.float64)
    A = np.empty((rows.size, n), dtype=np.float64)
    _load().orc_gemm_rows(fmt, _ptr(codes), _ptr(scales), _ptr(g), _ptr(X), _ptr(rows), rows.size, n, k,
                          _ptr(Y), _ptr(A))
    return Y, A


def moe_route(logits, topk, renorm):
    """(ids int32 [T][topk], weights fp64 [T][topk]) from fp32 router logits [T][E]:
    the topk largest logits (ties: lower index first), softmax weights, optionally
    renormalised over the selected experts."""
    logits = _c(logits, np.float32)
    tokens, experts = logits.shape
    ids = np.empty((tokens, topk), dtype=np.int32)
    w = np.empty((tokens, topk), dtype=np.float64)
    _load().orc_moe_route(_ptr(logits), tokens, experts, topk, int(renorm), _ptr(ids), _ptr(w))
    return ids, w


def silu(g: float) -> float:
    return _load().orc_silu(float(g))


def round_bf16(v: float) -> float:
    return _load().orc_round_bf16(float(v))


def moe_block(fmt, gu_codes, gu_scales, gu_g, dn_codes, dn_scales, dn_g, ids, w, x, experts, hidden, dff,
              rounding_tol=None):
    """(y, abs_y), both fp64 [T][hidden]: the MoE decode block (gate/up, SwiGLU to bf16,
    down, routing-weighted sum over the token's slots).

    With ``rounding_tol = (h_rel, h_abs, p_rel)`` it returns (y, abs_y, amb_y):
    amb_y bounds how far y may move when an implementation whose gate/up values
    are within h_rel * sum|w x| + h_abs (plus their own fp32 rounding) and whose
    fp32 SwiGLU is within p_rel relative rounds an activation to the other
    bf16 neighbour."""
    _check(fmt, hidden)
    _check(fmt, dff)
    gu_codes, gu_scales, gu_g = _c(gu_codes, np.uint8), _c(gu_scales, np.uint8), _c(gu_g, np.float32)
    dn_codes, dn_scales, dn_g = _c(dn_codes, np.uint8), _c(dn_scales, np.uint8), _c(dn_g, np.float32)
    ids, w, x = _c(ids, np.int32), _c(w, np.float32), _c(x, np.uint16)
    tokens, topk = ids.shape
    y = np.empty((tokens, hidden), dtype=np.float64)
    a = np.empty((tokens, hidden), dtype=np.float64)
    amb = None if rounding_tol is None else np.empty((tokens, hidden), dtype=np.float64)
    h_rel, h_abs, p_rel = (0.0, 0.0, 0.0) if rounding_tol is None else map(float, rounding_tol)
    _load().orc_moe_block(fmt, _ptr(gu_codes), _ptr(gu_scales), _ptr(gu_g), _ptr(dn_codes), _ptr(dn_scales),
                          _ptr(dn_g), _ptr(ids), _ptr(w), _ptr(x), experts, hidden, dff, tokens, topk,
                          h_rel, h_abs, p_rel, _ptr(y), _ptr(a), _ptr(amb))
    return (y, a) if amb is None else (y, a, amb)


def quantize(fmt, x, g, rows, k):
    """(codes, scales) of bf16 bits x [rows][k] (uint16): MX blocks of 32 with E8M0 scales
    (OCP MX conversion), NVFP4 blocks of 16 with E4M3 scales for the per-tensor scale g."""
    _check(fmt, k)
    x = _c(x, np.uint16)
    codes = np.zeros((rows, k if fmt == 2 else k // 2), dtype=np.uint8)
    scales = np.zeros((rows, k // (16 if fmt == 3 else 32)), dtype=np.uint8)
    _load().orc_quantize(fmt, _ptr(x), float(g if g is not None else 1.0), rows, k, _ptr(codes), _ptr(scales))
    return codes, scales


def requant_fp8(codes_in, tile_scales, n, k, bn=128, bk=128):
    """MXFP8 (codes uint8 [n][k], E8M0 scales uint8 [n][k/32]) of an FP8 block checkpoint: E4M3 codes
    uint8 [n][k] with one fp32 scale per bn x bk tile, tile_scales float32 [ceil(n/bn)][ceil(k/bk)]."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    codes_in = _c(codes_in, np.uint8)
    tile_scales = _c(tile_scales, np.float32)
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 32), dtype=np.uint8)
    _load().orc_requant_fp8(_ptr(codes_in), _ptr(tile_scales), n, k, bn, bk, _ptr(codes), _ptr(scales))
    return codes, scales


def split_e4m3(x, rows, k):
    """Two-term E4M3 split of bf16 bits x [rows][k] (uint16), per 32-element block:
    v = 2^e1 q1 + 2^e2 q2 + (remainder) with non-saturating scales (oracle.c).  Returns
    (q1, q2 uint8 [rows][k] E4M3 codes, e1, e2 uint8 [rows][k/32] E8M0 bytes)."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    x = _c(x, np.uint16)
    q1 = np.zeros((rows, k), dtype=np.uint8)
    q2 = np.zeros((rows, k), dtype=np.uint8)
    e1 = np.zeros((rows, k // 32), dtype=np.uint8)
    e2 = np.zeros((rows, k // 32), dtype=np.uint8)
    _load().orc_split_e4m3(_ptr(x), rows, k, _ptr(q1), _ptr(q2), _ptr(e1), _ptr(e2))
    return q1, q2, e1, e2


def within_tolerance(y_gpu, y_ref, abs_ref, rel=1e-5, atol=1e-6):
    """Boolean array: |y_gpu - y_ref| <= rel * abs_ref + atol (NaN matches NaN, equal infinities match)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    both_nan = np.isnan(y_gpu) & np.isnan(y_ref)
    with np.errstate(invalid="ignore"):
        ok = np.abs(y_gpu - y_ref) <= rel * abs_ref + atol
    return ok | both_nan | (y_gpu == y_ref)
