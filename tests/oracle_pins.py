"""Pin checks for the CPU oracle, written as plain functions so that the same
checks can run against the real oracle (tests/test_oracle_pins.py) and against
deliberately broken copies of it (tests/test_oracle_mutants.py).

Each check raises AssertionError on failure.  Sources of truth, none of them the
oracle itself: the stored E2M1 table, the E8M0 closed form 2^(u-127),
torch's float8_e4m3fn / float8_e8m0fnu / bfloat16 conversions, exact rational
brute force (tests/bruteforce.py), one-hot activations, closed-form sums and the
scale-bump invariant.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import bruteforce as bf
import oracle

MXFP4, MXFP8, NVFP4 = oracle.MXFP4, oracle.MXFP8, oracle.NVFP4
FMTS = (MXFP4, MXFP8, NVFP4)
BF16_ONE = 0x3F80


def _same_bits(a, b):
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return (a.view(np.uint32) == b.view(np.uint32)) | nan


def _rand_case(fmt, rng, n, k, exp_lo=118, exp_hi=130):
    if fmt == MXFP8:
        finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
        codes = finite[rng.integers(0, finite.size, size=(n, k))]
    else:
        codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    if fmt == NVFP4:
        scales = rng.integers(0x08, 0x7F, size=(n, k // 16), dtype=np.uint8)
        g = np.array([1.0 / 2688.0], dtype=np.float32)
    else:
        scales = rng.integers(exp_lo, exp_hi + 1, size=(n, k // 32), dtype=np.uint8)
        g = None
    f = rng.standard_normal(size=(2, k), dtype=np.float32)
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    return codes, scales, g, x


# ---- element formats -------------------------------------------------------------------

def check_e2m1_table():
    table = bf.e2m1_table()
    for c in range(16):
        v = oracle.e2m1(c)
        assert v == table[c] and math.copysign(1, v) == math.copysign(1, table[c]), (c, v, table[c])


def check_e8m0():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for u in range(255):
        assert oracle.e8m0(u) == 2.0 ** (u - 127) == ref[u], u
    assert math.isnan(oracle.e8m0(255)) and math.isnan(ref[255])


def check_e4m3():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = oracle.e4m3(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b] and math.copysign(1, v) == math.copysign(1, ref[b]), (b, v, ref[b])


def check_bf16():
    h = np.arange(0, 65536, 37, dtype=np.uint32)
    ref = torch.from_numpy(h.astype(np.int32)).to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    for hi, r in zip(h, ref):
        v = oracle.bf16(int(hi))
        assert (math.isnan(v) and math.isnan(r)) or v == r, hex(hi)


# ---- decode tiles ----------------------------------------------------------------------

def exhaustive_tile(fmt, g=None):
    """Every code against every scale byte: rows = scale bytes, columns = codes."""
    if fmt == MXFP8:
        k = 256
        codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    else:
        k = 32  # 16 codes, each twice: bytes c | c<<4
        row = np.array([c | (c << 4) for c in range(16)], dtype=np.uint8)
        codes = np.tile(row, (256, 1))
    bs = 16 if fmt == NVFP4 else 32
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k // bs, axis=1)
    gg = None if fmt != NVFP4 else np.array([g], dtype=np.float32)
    return codes, scales, gg, 256, k


def check_exhaustive_decode(fmt, g=1.0):
    codes, scales, gg, rows, k = exhaustive_tile(fmt, g)
    w = oracle.dequant(fmt, codes, scales, gg, rows, k)
    ref = bf.dequant(fmt, codes, scales, gg, rows, k)
    ok = _same_bits(w, ref)
    assert ok.all(), np.argwhere(~ok)[:5]


def check_random_decode(fmt, seed=1):
    rng = np.random.default_rng(seed)
    codes, scales, g, _ = _rand_case(fmt, rng, 4, 64, 0, 254)
    w = oracle.dequant(fmt, codes, scales, g, 4, 64)
    ref = bf.dequant(fmt, codes, scales, g, 4, 64)
    assert _same_bits(w, ref).all()


# ---- contraction -----------------------------------------------------------------------

def check_bruteforce_gemv(fmt, seed=0, n=4, k=32):
    rng = np.random.default_rng(seed)
    codes, scales, g, x = _rand_case(fmt, rng, n, k)
    y, a = oracle.gemv(fmt, codes, scales, g, x, n, k)
    ex = bf.gemv(fmt, codes, scales, g, x, n, k)
    for b in range(x.shape[0]):
        for r in range(n):
            assert bf.close(y[b, r], ex[b][r], k), (fmt, b, r, y[b, r], float(ex[b][r][0]))
            assert bf.close(a[b, r], (ex[b][r][1], ex[b][r][1]), k), (fmt, b, r)


def check_row_sweep(fmt):
    """One row holding every code, at three scales, x = N(0,1) bf16."""
    rng = np.random.default_rng(7)
    if fmt == MXFP8:
        k = 256
        codes = np.arange(256, dtype=np.uint8)[None, :].copy()
        codes[0, 0x7F] = 0x00
        codes[0, 0xFF] = 0x80
    else:
        k = 32
        codes = np.array([[(2 * i) | ((2 * i + 1) << 4) for i in range(8)] * 2], dtype=np.uint8)
    f = rng.standard_normal(size=(1, k), dtype=np.float32)
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    for u in ((120, 127, 134) if fmt != NVFP4 else (0x30, 0x38, 0x52)):
        bs = 16 if fmt == NVFP4 else 32
        scales = np.full((1, k // bs), u, dtype=np.uint8)
        g = None if fmt != NVFP4 else np.array([0.75], dtype=np.float32)
        y, _ = oracle.gemv(fmt, codes, scales, g, x, 1, k)
        ex = bf.gemv(fmt, codes, scales, g, x, 1, k)
        assert bf.close(y[0, 0], ex[0][0], k), (fmt, u)


def check_one_hot(fmt):
    """x = e_j  =>  y[r] = w[r][j] exactly, for j across a block boundary."""
    rng = np.random.default_rng(3)
    k = 64
    codes, scales, g, _ = _rand_case(fmt, rng, 8, k)
    w = bf.dequant(fmt, codes, scales, g, 8, k)
    for j in list(range(0, 34)) + [47, 48, 63]:
        x = np.zeros((1, k), dtype=np.uint16)
        x[0, j] = BF16_ONE
        y, a = oracle.gemv(fmt, codes, scales, g, x, 8, k)
        assert (y[0] == w[:, j].astype(np.float64)).all(), (fmt, j)
        assert (a[0] == np.abs(w[:, j]).astype(np.float64)).all(), (fmt, j)


def check_closed_form_sum():
    """MXFP4 codes all 1.0 (nibble 2), scale byte u: y = 2^(u-127) * sum(x), exactly."""
    rng = np.random.default_rng(11)
    k = 1024
    f = rng.standard_normal(size=(1, k), dtype=np.float32)
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    xs = [bf.bf16_value(int(h)) for h in x[0]]
    codes = np.full((3, k // 2), 0x22, dtype=np.uint8)
    for u in (127, 128, 100):
        scales = np.full((3, k // 32), u, dtype=np.uint8)
        y, _ = oracle.gemv(MXFP4, codes, scales, None, x, 3, k)
        assert (y[0] == math.fsum(xs) * 2.0 ** (u - 127)).all(), u


def check_scale_bump(fmt, seed=5):
    """Scale exponent of one block +1  =>  that block's contribution doubles exactly."""
    rng = np.random.default_rng(seed)
    k = 128
    codes, scales, g, x = _rand_case(fmt, rng, 4, k)
    bs = 16 if fmt == NVFP4 else 32
    cpb = bs if fmt == MXFP8 else bs // 2  # code bytes per block
    for b in range(k // bs):
        if fmt == NVFP4:
            e = (scales[:, b] >> 3) & 15
            if ((e < 1) | (e > 13)).any():
                scales[:, b] = (scales[:, b] & 0x87) | (7 << 3)
        iso = np.zeros_like(codes)
        iso[:, b * cpb:(b + 1) * cpb] = codes[:, b * cpb:(b + 1) * cpb]
        bumped = scales.copy()
        bumped[:, b] = scales[:, b] + (8 if fmt == NVFP4 else 1)
        y0, _ = oracle.gemv(fmt, iso, scales, g, x, 4, k)
        y1, _ = oracle.gemv(fmt, iso, bumped, g, x, 4, k)
        assert (y1 == 2.0 * y0).all(), (fmt, b)
        full0, a0 = oracle.gemv(fmt, codes, scales, g, x, 4, k)
        full1, _ = oracle.gemv(fmt, codes, bumped, g, x, 4, k)
        assert (np.abs((full1 - full0) - y0) <= 4 * k * 2.0 ** -53 * (a0 + np.abs(y0)) + 0.0).all(), (fmt, b)


def check_moe_bruteforce(fmt, x_per_slot):
    rng = np.random.default_rng(17)
    E, n, k, T, topk = 5, 3, 32, 3, 2
    if fmt == MXFP8:
        finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
        codes = finite[rng.integers(0, finite.size, size=(E, n, k))]
    else:
        codes = rng.integers(0, 256, size=(E, n, k // 2), dtype=np.uint8)
    bs = 16 if fmt == NVFP4 else 32
    if fmt == NVFP4:
        scales = rng.integers(0x08, 0x7F, size=(E, n, k // bs), dtype=np.uint8)
        g = (rng.random(E).astype(np.float32) + np.float32(0.25)).astype(np.float32)
    else:
        scales = rng.integers(118, 131, size=(E, n, k // bs), dtype=np.uint8)
        g = None
    ids = np.array([[0, 3], [3, 4], [-1, 5]], dtype=np.int32)  # repeats and two invalid ids
    shape = (T, topk, k) if x_per_slot else (T, k)
    f = rng.standard_normal(size=shape, dtype=np.float32)
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    y, a = oracle.moe_gemv(fmt, codes, scales, g, ids, x, x_per_slot, E, n, k)
    ex = bf.moe_gemv(fmt, codes, scales, g, ids, x, x_per_slot, E, n, k)
    for t in range(T):
        for s in range(topk):
            if ex[t][s] is None:
                assert np.isnan(y[t, s]).all()
                continue
            for r in range(n):
                assert bf.close(y[t, s, r], ex[t][s][r], k), (fmt, t, s, r)
                assert bf.close(a[t, s, r], (ex[t][s][r][1], ex[t][s][r][1]), k), (fmt, t, s, r)


def check_gemm_rows_bruteforce(fmt):
    rng = np.random.default_rng(23)
    m, n, k = 9, 5, 64
    codes, scales, g, _ = _rand_case(fmt, rng, n, k)
    f = rng.standard_normal(size=(m, k), dtype=np.float32)
    X = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    rows = np.array([0, 4, 8], dtype=np.int64)
    Y, A = oracle.gemm_rows(fmt, codes, scales, g, X, rows, n, k)
    g0 = None if g is None else g[0]
    for i, rr in enumerate(rows):
        for c in range(n):
            ex = bf.dot_exact(fmt, codes[c], scales[c], g0, X[rr], k)
            assert bf.close(Y[i, c], ex, k), (fmt, i, c)
            assert bf.close(A[i, c], (ex[1], ex[1]), k), (fmt, i, c)


def all_checks():
    """(name, callable) for every pin, used by the mutation test."""
    out = [("e2m1_table", check_e2m1_table), ("e8m0", check_e8m0), ("e4m3", check_e4m3),
           ("bf16", check_bf16), ("closed_form_sum", check_closed_form_sum)]
    for f in FMTS:
        out += [(f"exhaustive_decode_{f}", lambda f=f: check_exhaustive_decode(f)),
                (f"bruteforce_gemv_{f}", lambda f=f: check_bruteforce_gemv(f)),
                (f"row_sweep_{f}", lambda f=f: check_row_sweep(f)),
                (f"one_hot_{f}", lambda f=f: check_one_hot(f)),
                (f"scale_bump_{f}", lambda f=f: check_scale_bump(f)),
                (f"moe_{f}", lambda f=f: check_moe_bruteforce(f, 1)),
                (f"gemm_rows_{f}", lambda f=f: check_gemm_rows_bruteforce(f))]
    return out
