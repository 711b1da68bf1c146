"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random bytes, integers and normal samples; it holds none
of the block-float arithmetic (no decode, no scaling, no contraction).  Both the
CPU oracle and the HIP library receive exactly the arrays produced here.

Recipe (stated once, used everywhere):
  * numpy ``Generator(PCG64)``; each workload uses ``SeedSequence(seed).spawn(5)``
    child streams in the fixed order [codes, scales, x, ids, rows].
  * "uniform random 4-bit codes" = every code byte uniform on 0..255, i.e. both
    nibbles uniform on 0..15.
  * E8M0 scale bytes: integers uniform on an inclusive range [lo, hi].
  * E4M3 weight codes (MXFP8): uniform over the 254 finite encodings (every
    byte except 0x7F and 0xFF).
  * E4M3 block scales (NVFP4): uniform over the positive normal finite bytes
    0x08..0x7E; the per-tensor fp32 scale defaults to fp32(1/2688).
  * bf16 activations: fp32 standard normal samples rounded to bf16 with
    round-to-nearest-even (torch's fp32 -> bf16 conversion); returned as the
    raw uint16 bit patterns.
  * MoE routing: per token, ``topk`` distinct expert ids drawn uniformly
    (``choice(E, topk, replace=False)``).
  * Router logits: fp32 standard normal samples.
  * MoE block: the gate/up bank [E][2*dff][hidden] is drawn first, then the
    down bank [E][hidden][dff], from the same codes and scales streams; routing
    weights are fp32 uniform on [0.1, 1.1) divided by topk, from the rows stream.
  * "Exact" gate/up inputs (every partial sum of the gate/up products is an
    fp32 number, whatever the summation order): activations are integers
    uniform on [-2, 2]; MX block scales uniform on [122, 125]; MXFP8 codes
    with exponent field 5..8 (magnitudes 0.25 .. 3.75, any sign and
    mantissa); NVFP4 block-scale bytes with exponent field 6..8
    (0.5 .. 3.75) and per-tensor scales 2^-11 (so that every decoded NVFP4
    weight is an fp32 number too).
"""
from __future__ import annotations

import numpy as np

MXFP4, MXFP8, NVFP4 = 1, 2, 3
FORMATS = {"mxfp4": MXFP4, "mxfp8": MXFP8, "nvfp4": NVFP4}
BLOCK = {MXFP4: 32, MXFP8: 32, NVFP4: 16}

# E4M3 byte values that encode a finite number (0x7F and 0xFF are NaN).
_E4M3_FINITE = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
NVFP4_DEFAULT_GLOBAL = np.float32(1.0 / 2688.0)


def streams(seed: int = 0):
    """Five independent generators in the order [codes, scales, x, ids, rows]."""
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(5)]


def code_bytes_per_row(fmt: int, k: int) -> int:
    return k if fmt == MXFP8 else k // 2


def bf16_normal(rng, shape) -> np.ndarray:
    """N(0,1) fp32 samples rounded (RNE) to bf16, as uint16 bit patterns."""
    import torch

    f = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _e4m3_with_exponent(lo: int, hi: int) -> np.ndarray:
    """E4M3 bytes whose 4-bit exponent field (bits 6..3) lies in [lo, hi], any sign and mantissa."""
    return np.array([b for b in range(256) if lo <= (b >> 3) & 0xF <= hi and b not in (0x7F, 0xFF)],
                    dtype=np.uint8)


def weights(fmt: int, rng_codes, rng_scales, rows: int, k: int, exp_lo: int = 118, exp_hi: int = 130,
            experts: int | None = None, fp8_exp: tuple | None = None, nv_scale_exp: tuple | None = None):
    """Packed codes, block scales and (NVFP4) per-tensor scale for a [rows][k] weight.

    With ``experts`` set the arrays get a leading expert dimension (an MoE bank).
    ``fp8_exp`` / ``nv_scale_exp`` restrict MXFP8 codes / NVFP4 block-scale bytes
    to an exponent-field range.
    Returns (codes uint8, scales uint8, global_scale float32 array or None).
    """
    lead = () if experts is None else (experts,)
    bs = BLOCK[fmt]
    if fmt == MXFP8:
        pool = _E4M3_FINITE if fp8_exp is None else _e4m3_with_exponent(*fp8_exp)
        idx = rng_codes.integers(0, pool.size, size=lead + (rows, k))
        codes = pool[idx]
    else:
        codes = rng_codes.integers(0, 256, size=lead + (rows, k // 2), dtype=np.uint8)
    if fmt == NVFP4:
        if nv_scale_exp is None:
            scales = rng_scales.integers(0x08, 0x7F, size=lead + (rows, k // bs), dtype=np.uint8)
        else:
            pool = np.array([b for b in _e4m3_with_exponent(*nv_scale_exp) if b < 0x80], dtype=np.uint8)
            scales = pool[rng_scales.integers(0, pool.size, size=lead + (rows, k // bs))]
        g = np.full(lead if lead else (1,), NVFP4_DEFAULT_GLOBAL, dtype=np.float32)
    else:
        scales = rng_scales.integers(exp_lo, exp_hi + 1, size=lead + (rows, k // bs), dtype=np.uint8)
        g = None
    return np.ascontiguousarray(codes, dtype=np.uint8), np.ascontiguousarray(scales, dtype=np.uint8), g


def int_bf16(rng, shape, lim: int) -> np.ndarray:
    """Integers uniform on [-lim, lim] as bf16 bit patterns (exact in bf16 for lim <= 256)."""
    import torch

    f = rng.integers(-lim, lim + 1, size=shape).astype(np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def router_logits(rng, tokens: int, experts: int) -> np.ndarray:
    """fp32 [tokens][experts] standard normal router logits."""
    return rng.standard_normal(size=(tokens, experts), dtype=np.float32)


def moe_ids(rng, tokens: int, topk: int, experts: int) -> np.ndarray:
    """int32 [tokens][topk], each row ``topk`` distinct ids uniform on [0, experts)."""
    return np.stack([rng.choice(experts, size=topk, replace=False) for _ in range(tokens)]).astype(np.int32)


def row_subset(rng, m: int, count: int) -> np.ndarray:
    """``count`` distinct row indices of [0, m), sorted, int64."""
    return np.sort(rng.choice(m, size=count, replace=False)).astype(np.int64)


# ---- the five workloads -----------------------------------------------------------------

def single_gemv(seed: int = 0):
    """MXFP4 GEMV, 512 rows x K=1024, E8M0 exponents U[120,130], one bf16 vector."""
    sc, ss, sx, _, _ = streams(seed)
    codes, scales, _ = weights(MXFP4, sc, ss, 512, 1024, 120, 130)
    x = bf16_normal(sx, (1, 1024))
    return dict(fmt=MXFP4, codes=codes, scales=scales, g=None, x=x, n=512, k=1024)


DENSE_SHAPES = {"gate_up": (51200, 5120), "down": (5120, 25600), "qkv": (7168, 5120)}


def dense_layer(which: str, batch: int, seed: int = 0, fmt: int = MXFP4):
    """One projection of the dense 30B-class decode layer (E8M0 exponents U[118,130])."""
    n, k = DENSE_SHAPES[which]
    sc, ss, sx, _, _ = streams(seed)
    codes, scales, g = weights(fmt, sc, ss, n, k, 118, 130)
    x = bf16_normal(sx, (batch, k))
    return dict(fmt=fmt, codes=codes, scales=scales, g=g, x=x, n=n, k=k)


MOE_SHAPES = {"gate_up": (1536, 2048), "down": (2048, 768)}
MOE_EXPERTS, MOE_TOPK = 128, 8


def moe_layer(which: str, tokens: int, seed: int = 0, fmt: int = MXFP4, experts: int = MOE_EXPERTS,
              topk: int = MOE_TOPK):
    """Expert bank + routing for the 30B-A3B-like MoE layer (128 experts, top-8)."""
    n, k = MOE_SHAPES[which]
    sc, ss, sx, si, _ = streams(seed)
    codes, scales, g = weights(fmt, sc, ss, n, k, 118, 130, experts=experts)
    ids = moe_ids(si, tokens, topk, experts)
    per_slot = which == "down"
    x = bf16_normal(sx, (tokens, topk, k) if per_slot else (tokens, k))
    return dict(fmt=fmt, codes=codes, scales=scales, g=g, ids=ids, x=x, x_per_slot=int(per_slot),
                experts=experts, n=n, k=k, tokens=tokens, topk=topk)


def moe_block(tokens: int, seed: int = 0, fmt: int = MXFP4, experts: int = MOE_EXPERTS, hidden: int = 2048,
              dff: int = 768, topk: int = MOE_TOPK, exact: bool = False):
    """One MoE decode block (gate/up bank, down bank, routing, activations) of the
    30B-A3B-like layer: hidden 2048, expert width 768, 128 experts, top-8.  With
    ``exact`` the gate/up inputs make every gate/up sum an fp32 number."""
    sc, ss, sx, si, sr = streams(seed)
    if exact:
        gu = weights(fmt, sc, ss, 2 * dff, hidden, 122, 125, experts=experts, fp8_exp=(5, 8), nv_scale_exp=(6, 8))
        if fmt == NVFP4:
            gu = (gu[0], gu[1], np.full(experts, 2.0 ** -11, dtype=np.float32))
        x = int_bf16(sx, (tokens, hidden), 2)
    else:
        gu = weights(fmt, sc, ss, 2 * dff, hidden, 118, 130, experts=experts)
        x = bf16_normal(sx, (tokens, hidden))
    dn = weights(fmt, sc, ss, hidden, dff, 118, 130, experts=experts)
    ids = moe_ids(si, tokens, topk, experts)
    w = ((sr.random((tokens, topk), dtype=np.float32) + np.float32(0.1)) / np.float32(topk)).astype(np.float32)
    return dict(fmt=fmt, gu=gu, dn=dn, ids=ids, w=w, x=x, experts=experts, hidden=hidden, dff=dff,
                tokens=tokens, topk=topk)


def format_sweep(fmt: int, seed: int = 0):
    """Dense down shape (5120 x 25600), batch 1, in the given format."""
    return dense_layer("down", 1, seed=seed, fmt=fmt)


def prefill(seed: int = 0, m: int = 4096, n: int = 25600, k: int = 5120, checked_rows: int = 64, fmt: int = MXFP4):
    """bf16 token rows x block-float weight (E8M0 U[120,130]; NVFP4: the default
    E4M3 scales and per-tensor scale) plus the seeded rows the oracle checks."""
    sc, ss, sx, _, sr = streams(seed)
    codes, scales, g = weights(fmt, sc, ss, n, k, 120, 130)
    x = bf16_normal(sx, (m, k))
    rows = row_subset(sr, m, checked_rows)
    return dict(fmt=fmt, codes=codes, scales=scales, g=g, x=x, m=m, n=n, k=k, rows=rows)
