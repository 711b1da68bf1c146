"""Exact rational brute force for tiny block-float GEMV / MoE / GEMM cases.

Written independently of the C oracle: element values come from the stored
E2M1 table (tests/golden/e2m1_table.txt), from 2**(u-127) for E8M0 and from
torch's ``float8_e4m3fn`` conversion for E4M3; products and sums are exact
``fractions.Fraction`` arithmetic.  Only for inputs of a few hundred elements.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

MXFP4, MXFP8, NVFP4 = 1, 2, 3
_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e2m1_table.txt")


def e2m1_table():
    """{code: float} from the stored table (value strings like '-0' keep their sign)."""
    table = {}
    with open(_GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            table[int(code)] = float(val)
    assert sorted(table) == list(range(16))
    return table


_E2M1 = e2m1_table()
_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_value(b: int) -> float:
    return float(_E4M3[b])


def bf16_value(h: int) -> float:
    return float(torch.tensor([h], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64)[0])


def _frac(v: float):
    """Fraction of a finite float, or the float itself (inf / nan) otherwise."""
    return Fraction(v) if np.isfinite(v) else v


def code_at(fmt, codes_row, j):
    if fmt == MXFP8:
        return int(codes_row[j])
    byte = int(codes_row[j // 2])
    return byte & 0xF if j % 2 == 0 else byte >> 4


def weight_fp32(fmt, codes_row, scales_row, g, j) -> np.float32:
    """Decoded element as np.float32: the exact product, rounded once."""
    c = code_at(fmt, codes_row, j)
    q = e4m3_value(c) if fmt == MXFP8 else _E2M1[c]
    if fmt == NVFP4:
        s = e4m3_value(int(scales_row[j // 16]))
        gf = float(np.float32(g))
        if not (np.isfinite(q) and np.isfinite(s)):
            return np.float32(np.nan)
        exact = Fraction(q) * Fraction(s) * Fraction(gf)
        negative_zero = bool(np.signbit(q) ^ np.signbit(s) ^ np.signbit(gf))
    else:
        u = int(scales_row[j // 32])
        if u == 255 or not np.isfinite(q):
            return np.float32(np.nan)
        exact = Fraction(q) * Fraction(2) ** (u - 127)
        negative_zero = bool(np.signbit(q))
    with np.errstate(over="ignore"):
        v = np.float32(float(abs(exact))) if abs(exact) < Fraction(2) ** 1000 else np.float32(np.inf)
    if exact < 0 or (exact == 0 and negative_zero):
        v = -v
    return v


def dequant(fmt, codes, scales, g, rows, k):
    g0 = None if g is None else np.asarray(g, dtype=np.float32).reshape(-1)[0]
    out = np.empty((rows, k), dtype=np.float32)
    for r in range(rows):
        for j in range(k):
            out[r, j] = weight_fp32(fmt, codes[r], scales[r], g0, j)
    return out


def dot_exact(fmt, codes_row, scales_row, g, x_row, k):
    """(exact sum, exact sum of |terms|) as Fractions (or float inf/nan)."""
    acc, aacc = Fraction(0), Fraction(0)
    for j in range(k):
        w = float(weight_fp32(fmt, codes_row, scales_row, g, j))
        xv = bf16_value(int(x_row[j]))
        t = _frac(w) * _frac(xv) if np.isfinite(w) and np.isfinite(xv) else w * xv
        acc = acc + t
        aacc = aacc + abs(t)
    return acc, aacc


def gemv(fmt, codes, scales, g, x, n, k):
    g0 = None if g is None else np.asarray(g, dtype=np.float32).reshape(-1)[0]
    x = np.asarray(x).reshape(-1, k)
    return [[dot_exact(fmt, codes[r], scales[r], g0, x[b], k) for r in range(n)] for b in range(x.shape[0])]


def moe_gemv(fmt, codes, scales, g, ids, x, x_per_slot, experts, n, k):
    tokens, topk = ids.shape
    out = []
    for t in range(tokens):
        slots = []
        for s in range(topk):
            e = int(ids[t, s])
            xv = x[t, s] if x_per_slot else x[t]
            if not 0 <= e < experts:
                slots.append(None)
                continue
            ge = None if g is None else np.asarray(g, dtype=np.float32)[e]
            slots.append([dot_exact(fmt, codes[e, r], scales[e, r], ge, xv, k) for r in range(n)])
        out.append(slots)
    return out


def close(y, exact_pair, k):
    """Oracle fp64 y against the exact sum: within k * 2^-53 * sum|terms| (sequential fp64 bound)."""
    exact, aexact = exact_pair
    if not isinstance(exact, Fraction):
        return (np.isnan(exact) and np.isnan(y)) or exact == y
    bound = Fraction(k) * Fraction(1, 2 ** 53) * aexact
    return abs(Fraction(y) - exact) <= bound
