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


# ---- MoE decode block -------------------------------------------------------------

def _route_reference(logits, topk, renorm):
    """Pure-Python routing: order experts by (-logit, index), softmax with math.exp."""
    ids, ws = [], []
    for row in logits.astype(np.float64):
        order = sorted(range(row.size), key=lambda e: (-row[e], e))[:topk]
        mx = max(row)
        den = math.fsum(math.exp(v - mx) for v in row)
        w = [math.exp(row[e] - mx) / den for e in order]
        if renorm:
            tot = math.fsum(w)
            w = [v / tot for v in w]
        ids.append(order)
        ws.append(w)
    return np.array(ids, dtype=np.int32), np.array(ws, dtype=np.float64)


def check_route():
    rng = np.random.default_rng(31)
    for topk in (1, 2, 4, 6):
        for renorm in (False, True):
            logits = rng.standard_normal(size=(4, 6)).astype(np.float32)
            logits[1, 2] = logits[1, 4] = logits[1].max() + np.float32(1.0)  # tie at the top
            logits[2, :] = np.float32(0.5)                                     # all equal
            ids, w = oracle.moe_route(logits, topk, renorm)
            ids_r, w_r = _route_reference(logits, topk, renorm)
            assert (ids == ids_r).all(), (topk, renorm, ids, ids_r)
            assert np.allclose(w, w_r, rtol=1e-14, atol=0.0), (topk, renorm)
            if renorm:
                assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def check_silu():
    assert oracle.silu(0.0) == 0.0
    for g in (0.25, 1.0, 3.5, 17.0):
        # silu(-g) = -g * sigmoid(-g) = silu(g) - g
        assert abs(oracle.silu(-g) - (oracle.silu(g) - g)) <= 1e-15 * max(1.0, g), g
        assert abs(oracle.silu(g) - g / (1.0 + math.exp(-g))) <= 1e-16 * g
    assert oracle.silu(60.0) == 60.0 * (1.0 / (1.0 + math.exp(-60.0)))
    assert 0.0 > oracle.silu(-60.0) > -1e-20


def check_round_bf16():
    rng = np.random.default_rng(37)
    f = np.concatenate([rng.standard_normal(4000).astype(np.float32) * np.float32(1e3),
                        (np.arange(1, 512, dtype=np.float32) * np.float32(2.0 ** -8) + np.float32(1.0)),  # halfway points
                        np.array([1e-39, -3e-40, 3.3e38, -3.39e38, 2.0 ** -133, 1.0 + 2.0 ** -8], dtype=np.float32)])
    ref = torch.from_numpy(f).to(torch.bfloat16).float().numpy()
    got = np.array([oracle.round_bf16(float(v)) for v in f])
    assert (got == ref.astype(np.float64)).all(), np.argwhere(got != ref)[:5]


def _moe_block_case(fmt, seed, E=5, H=64, dff=32, T=3, topk=2):
    rng = np.random.default_rng(seed)
    gu_codes, gu_scales, gu_g, _ = _rand_case(fmt, rng, E * 2 * dff, H)
    dn_codes, dn_scales, dn_g, _ = _rand_case(fmt, rng, E * H, dff)
    if fmt == NVFP4:
        gu_g = (rng.random(E).astype(np.float32) + np.float32(0.25)).astype(np.float32)
        dn_g = (rng.random(E).astype(np.float32) + np.float32(0.25)).astype(np.float32)
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random(size=(T, topk)).astype(np.float32) + np.float32(0.1)
    f = rng.standard_normal(size=(T, H), dtype=np.float32)
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    return dict(gu=(gu_codes.reshape(E, 2 * dff, -1), gu_scales.reshape(E, 2 * dff, -1), gu_g),
                dn=(dn_codes.reshape(E, H, -1), dn_scales.reshape(E, H, -1), dn_g),
                ids=ids, w=w, x=x, E=E, H=H, dff=dff, T=T, topk=topk)


def _moe_block_composed(fmt, c):
    """The block from already-pinned pieces: the MoE GEMV for gate/up and down, and
    numpy / torch for the SwiGLU and its bf16 rounding."""
    E, H, dff, T, topk = c["E"], c["H"], c["dff"], c["T"], c["topk"]
    h, _ = oracle.moe_gemv(fmt, *c["gu"], c["ids"], c["x"], 0, E, 2 * dff, H)
    h32 = h.astype(np.float32)
    g, u = h32[..., :dff], h32[..., dff:]
    with np.errstate(over="ignore", invalid="ignore"):
        g64 = g.astype(np.float64)
        silu32 = (g64 / (1.0 + np.exp(-g64))).astype(np.float32)   # silu rounded to fp32
        act = torch.from_numpy(silu32 * u).to(torch.bfloat16)        # fp32 product, then RNE to bf16
    a_bits = act.view(torch.int16).numpy().view(np.uint16).copy()
    yd, ad = oracle.moe_gemv(fmt, *c["dn"], c["ids"], a_bits, 1, E, H, dff)
    w = c["w"].astype(np.float64)[..., None]
    return (w * yd).sum(axis=1), (np.abs(w) * ad).sum(axis=1)


def check_moe_block(fmt, seed=41):
    c = _moe_block_case(fmt, seed)
    y, a = oracle.moe_block(fmt, *c["gu"], *c["dn"], c["ids"], c["w"], c["x"], c["E"], c["H"], c["dff"])
    y_c, a_c = _moe_block_composed(fmt, c)
    assert np.isfinite(y).all()
    assert (np.abs(y - y_c) <= 1e-12 * a_c).all(), np.abs(y - y_c).max()
    assert (np.abs(a - a_c) <= 1e-12 * a_c).all()
    bad = c["ids"].copy()
    bad[1, 0] = c["E"]
    y2, _ = oracle.moe_block(fmt, *c["gu"], *c["dn"], bad, c["w"], c["x"], c["E"], c["H"], c["dff"])
    assert np.isnan(y2[1]).all() and np.isfinite(y2[0]).all() and np.isfinite(y2[2]).all()


def _one_block(fmt, gate_row0, up_row0, x_vals, H=32, dff=32):
    """A one-expert MXFP4 block: gate row 0 and up row 0 (rows 0 and dff of the
    gate/up bank) as given lists of (element, code, scale byte), x from exact
    bf16 values, the down row 0 equal to 1.0 on element 0; every other weight 0."""
    gc = np.zeros((1, 2 * dff, H // 2), dtype=np.uint8)
    gs = np.full((1, 2 * dff, H // 32), 127, dtype=np.uint8)
    for row, elems in ((0, gate_row0), (dff, up_row0)):
        for k, code, scale in elems:
            gc[0, row, k // 2] |= code << (4 * (k % 2))     # element 2i: low nibble
            gs[0, row, k // 32] = scale
    dc = np.zeros((1, H, dff // 2), dtype=np.uint8)
    ds = np.full((1, H, dff // 32), 127, dtype=np.uint8)
    dc[0, 0, 0] = 0x02                                        # W_dn[0][0] = 1.0
    f = np.zeros((1, H), dtype=np.float32)
    f[0, :len(x_vals)] = x_vals
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    ids = np.zeros((1, 1), dtype=np.int32)
    w = np.ones((1, 1), dtype=np.float32)
    y, _ = oracle.moe_block(fmt, gc, gs, None, dc, ds, None, ids, w, x, 1, H, dff)
    return y[0]


def check_swiglu_tie():
    """Gate g = 32 (E2M1 4.0 at scale 2^3), x = (1, 2^-7, 2^-8): silu(32) is 32 in
    fp32, so a = bf16(32 u) with u = 2^-5 (1 + 2^-7 + 2^-8) (three E2M1 1.0 at
    scale 2^-5) is 1 + 2^-7 + 2^-8, exactly halfway between the bf16 numbers
    1 + 2^-7 and 1 + 2^-6: ties to even give 1 + 2^-6.  With one more 2^-8 dropped
    (u = 2^-5 (1 + 2^-8)) the tie is between 1 and 1 + 2^-7: even is 1.
    y[0] = a (one expert, weight 1, W_dn row 0 = e_0); every other y is 0."""
    gate = [(0, 0x6, 130)]
    xv = [1.0, 2.0 ** -7, 2.0 ** -8]
    y = _one_block(MXFP4, gate, [(0, 0x2, 122), (1, 0x2, 122), (2, 0x2, 122)], xv)
    assert y[0] == 1.0 + 2.0 ** -6 and (y[1:] == 0).all(), y[:4]
    y = _one_block(MXFP4, gate, [(0, 0x2, 122), (2, 0x2, 122)], xv)
    assert y[0] == 1.0, y[0]
    y = _one_block(MXFP4, gate, [(0, 0xA, 122), (1, 0xA, 122), (2, 0xA, 122)], xv)  # sign bit: u < 0
    assert y[0] == -(1.0 + 2.0 ** -6), y[0]
    y = _one_block(MXFP4, [(0, 0xE, 130)], [(0, 0x2, 122)], xv)                       # g = -32: silu ~ -4e-13
    assert y[0] <= 0.0 and abs(y[0]) < 1e-12, y[0]


def _block_fp32(c, rounding="rne"):
    """The block as an fp32 implementation computes it (torch on the CPU, its own
    summation order, silu as g / (1 + exp(-g)) in fp32), MXFP4 weights decoded by
    the pinned dequantiser.  ``rounding``: "rne" (correct), "trunc" or "none"
    (planted mistakes in the activation rounding)."""
    E, H, dff = c["experts"], c["hidden"], c["dff"]
    gc, gs, _ = c["gu"]
    dc, ds, _ = c["dn"]
    Wgu = torch.from_numpy(oracle.dequant(MXFP4, gc.reshape(E * 2 * dff, -1), gs.reshape(E * 2 * dff, -1), None,
                                          E * 2 * dff, H)).reshape(E, 2 * dff, H)
    Wdn = torch.from_numpy(oracle.dequant(MXFP4, dc.reshape(E * H, -1), ds.reshape(E * H, -1), None,
                                          E * H, dff)).reshape(E, H, dff)
    x = torch.from_numpy(c["x"].view(np.int16)).view(torch.bfloat16).float()
    y = torch.zeros(c["tokens"], H)
    for t in range(c["tokens"]):
        for s in range(c["topk"]):
            e = int(c["ids"][t, s])
            h = Wgu[e] @ x[t]
            g, u = h[:dff], h[dff:]
            p = g / (1.0 + torch.exp(-g)) * u
            if rounding == "rne":
                a = p.to(torch.bfloat16).float()
            elif rounding == "trunc":
                a = (p.view(torch.int32) & ~0xFFFF).view(torch.float32)
            else:
                a = p
            y[t] += float(c["w"][t, s]) * (Wdn[e] @ a)
    return y.double().numpy()


ROUNDING_TOL_EXACT = (0.0, 0.0, 2.0 ** -21)      # gate/up exact; fp32 SwiGLU within 8 ulp
ROUNDING_TOL_CONTRACT = (1e-5, 1e-6, 2.0 ** -21)  # gate/up within the GEMV acceptance bound


def check_block_rounding_bound():
    """amb_y covers an fp32 implementation's choice of bf16 neighbour and no more
    than that: the correct fp32 block passes |y - y_ref| <= 1e-5 abs + amb + 1e-6,
    truncated or unrounded activations fail it; amb is 0 when nothing is uncertain."""
    import synth
    for exact, tol in ((True, ROUNDING_TOL_EXACT), (False, ROUNDING_TOL_CONTRACT)):
        c = synth.moe_block(4, seed=17, experts=6, hidden=512, dff=256, topk=4, exact=exact)
        args = (MXFP4, *c["gu"], *c["dn"], c["ids"], c["w"], c["x"], c["experts"], c["hidden"], c["dff"])
        y, a, amb = oracle.moe_block(*args, rounding_tol=tol)
        y0, a0, amb0 = oracle.moe_block(*args, rounding_tol=(0.0, 0.0, 0.0))
        assert (y0 == y).all() and (a0 == a).all() and (amb0 == 0).all()
        assert (amb >= 0).all() and np.isfinite(amb).all()
        bound = 1e-5 * a + amb + 1e-6
        assert (np.abs(_block_fp32(c) - y) <= bound).all(), exact
        for bad in ("trunc", "none"):
            assert (np.abs(_block_fp32(c, bad) - y) > bound).sum() > y.size // 10, (exact, bad)
        if exact:
            assert np.median(amb / a) < 1e-7


def check_block_rounding_bound_bruteforce(seed=43, p_rel=2.0 ** -10):
    """amb_y against brute force.  A one-expert MXFP4 block (hidden 32, expert width
    32, one token, weight w) whose gate/up values are exact in fp32 (h_rel = h_abs =
    0), so an activation's legitimate values are the bf16 roundings of every value
    within p_rel * |p| of its fp32 product p.  From pinned pieces (the oracle's MoE
    GEMV, numpy's fp32 SwiGLU, torch's bf16 rounding) the test lists each
    activation's candidates, enumerates every combination of them, and takes the
    largest |y(combination) - y| per output: amb_y must cover it everywhere and equal
    it on output 0, whose down row is built so that every activation's other
    candidate moves y the same way."""
    rng = np.random.default_rng(seed)
    H = dff = 32
    gc = rng.integers(0, 256, size=(1, 2 * dff, H // 2), dtype=np.uint8)
    gs = rng.integers(124, 127, size=(1, 2 * dff, 1), dtype=np.uint8)
    # x: small integers, so that every gate/up sum is an fp32 number (exact in any order)
    f = rng.integers(-3, 4, size=(1, H)).astype(np.float32)
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    ids = np.zeros((1, 1), dtype=np.int32)
    w = np.array([[0.75]], dtype=np.float32)
    h, _ = oracle.moe_gemv(MXFP4, gc, gs, None, ids, x, 0, 1, 2 * dff, H)
    h32 = h[0, 0].astype(np.float32)
    assert (h32.astype(np.float64) == h[0, 0]).all()              # premise: gate/up exact in fp32
    g, u = h32[:dff].astype(np.float64), h32[dff:]
    p = ((g / (1.0 + np.exp(-g))).astype(np.float32) * u).astype(np.float64)   # fp32 SwiGLU product
    rne = lambda v: torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.bfloat16).double().numpy()
    a = rne(p)
    lo, hi = rne(p - p_rel * np.abs(p)), rne(p + p_rel * np.abs(p))
    cands = []
    for j in range(dff):
        # every bf16 value from lo to hi (rounding is monotone): step through the bf16 grid
        c, v = [], torch.tensor([lo[j]], dtype=torch.float64).to(torch.bfloat16)
        while float(v) <= hi[j]:
            c.append(float(v))
            v = torch.nextafter(v, torch.tensor([np.inf], dtype=torch.bfloat16))
        cands.append(c)
    unsure = [j for j in range(dff) if len(cands[j]) > 1]
    assert 6 <= len(unsure) <= 16, len(unsure)                     # premise: enough choices to matter
    # down bank: row 0 = the sign of each unsure activation's other candidate, random rows otherwise
    dcodes = rng.integers(0, 256, size=(1, H, dff // 2), dtype=np.uint8)
    dcodes[0, 0, :] = 0
    for j in unsure:
        other = max(cands[j], key=lambda v: abs(v - a[j]))
        code = 0x2 if other > a[j] else 0xA                        # E2M1 +1 / -1
        dcodes[0, 0, j // 2] |= code << (4 * (j % 2))
    dscales = np.full((1, H, 1), 127, dtype=np.uint8)
    Wdn = oracle.dequant(MXFP4, dcodes[0], dscales[0], None, H, dff).astype(np.float64)
    y, _, amb = oracle.moe_block(MXFP4, gc, gs, None, dcodes, dscales, None, ids, w, x, 1, H, dff,
                                 rounding_tol=(0.0, 0.0, p_rel))
    ya = float(w[0, 0]) * (Wdn @ a)                               # fp64, its own summation order
    assert (np.abs(y[0] - ya) <= 1e-14 * float(w[0, 0]) * (np.abs(Wdn) @ np.abs(a))).all()
    # every combination of candidates
    combos = np.array(np.meshgrid(*[cands[j] for j in unsure], indexing="ij")).reshape(len(unsure), -1).T
    A = np.tile(a, (combos.shape[0], 1))
    A[:, unsure] = combos
    ys = float(w[0, 0]) * (A @ Wdn.T)
    worst = np.abs(ys - y[0]).max(axis=0)
    assert (amb[0] >= worst * (1 - 1e-12)).all(), (amb[0], worst)
    assert abs(amb[0, 0] - worst[0]) <= 1e-12 * worst[0] and worst[0] > 0, (amb[0, 0], worst[0])


# ---- block-float quantizer ---------------------------------------------------------------
# An independent reference: element values from the stored E2M1 table and torch's E4M3
# decoder, the nearest value found by exhaustive search (ties: even code), the MX scale
# exponent from math.frexp, the NVFP4 arithmetic in numpy float32.

def _grid(fmt_elem):
    """[(value, code)] of the non-negative finite codes of E2M1 ("e2m1") or E4M3 ("e4m3")."""
    if fmt_elem == "e2m1":
        table = bf.e2m1_table()
        return [(table[c], c) for c in range(8)]
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().tolist()
    return [(v, c) for c, v in enumerate(vals)]


def _nearest(a, grid):
    """Code of the grid value nearest to a >= 0; ties to the even code; above the top: the top."""
    top = max(grid)
    if a >= top[0]:
        return top[1]
    best = None
    for v, c in grid:
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def _quantize_reference(fmt, xbits, g):
    f = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    rows, k = f.shape
    bs = 16 if fmt == NVFP4 else 32
    e2m1, e4m3 = _grid("e2m1"), _grid("e4m3")
    codes = np.zeros((rows, k), dtype=np.int64)
    scales = np.zeros((rows, k // bs), dtype=np.uint8)
    for r in range(rows):
        for b in range(k // bs):
            blk = f[r, b * bs:(b + 1) * bs]
            amax = float(np.max(np.abs(blk)))
            if fmt == NVFP4:
                t = float(np.float32(amax) / (np.float32(6.0) * np.float32(g)))
                sc = _nearest(t, e4m3)
                scales[r, b] = sc
                s_val = dict((c, v) for v, c in e4m3)[sc]
                den = np.float32(np.float32(s_val) * np.float32(g))
                with np.errstate(over="ignore"):  # an overflowing quotient saturates
                    ps = [0.0 if s_val == 0 else float(np.float32(v) / den) for v in blk]
            else:
                emax = 2 if fmt == MXFP4 else 8
                se = -127 if amax == 0 else min(127, max(-127, math.frexp(amax)[1] - 1 - emax))
                scales[r, b] = se + 127
                ps = [v / 2.0 ** se for v in blk]
            for j, pv in enumerate(ps):
                neg = int(xbits[r, b * bs + j]) >> 15
                if fmt == MXFP8:
                    codes[r, b * bs + j] = _nearest(abs(pv), e4m3) | (neg << 7)
                else:
                    codes[r, b * bs + j] = _nearest(abs(pv), e2m1) | (neg << 3)
    if fmt != MXFP8:
        codes = (codes[:, 0::2] | (codes[:, 1::2] << 4))
    return codes.astype(np.uint8), scales


def _bits(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _quant_cases(fmt, seed):
    rng = np.random.default_rng(seed)
    bs = 16 if fmt == NVFP4 else 32
    rows = []
    # random magnitudes spread over many binades, both signs
    for _ in range(6):
        rows.append((rng.standard_normal(2 * bs) * np.exp2(rng.integers(-20, 20, size=2 * bs))).tolist())
    # exact ties of the element grids, with the block maximum fixing the scale
    if fmt == MXFP8:
        ties = [256.0, 1.0625, 1.1875, 3.0 * 2 ** -10, 2 ** -10, -1.0625, 0.0, -0.0, 300.0, 2 ** -11]
    else:
        ties = [5.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -0.25, -5.0, 0.0, -0.0, 0.1, 4.9]
    rows.append((ties * (2 * bs // len(ties) + 1))[:2 * bs])
    rows.append([0.0] * (2 * bs))                                       # zero blocks
    rows.append([1e-39, -2e-40] + [0.0] * (2 * bs - 2))                 # bf16 subnormals: scale clamp
    rows.append([3.0e38] + [1.0] * (2 * bs - 1))                        # near the top of bf16
    return _bits(rows)


def check_quantize_nearest(fmt):
    x = _quant_cases(fmt, 7 + fmt)
    g = float(np.float32(1.0 / 2688.0)) if fmt == NVFP4 else None
    rows, k = x.shape
    for gg in ([g, float(np.float32(0.75)), float(np.float32(3.0e-3))] if fmt == NVFP4 else [None]):
        codes, scales = oracle.quantize(fmt, x, gg, rows, k)
        rc, rs = _quantize_reference(fmt, x, gg)
        assert (scales == rs).all(), (fmt, gg, np.argwhere(scales != rs)[:3])
        assert (codes == rc).all(), (fmt, gg, np.argwhere(codes != rc)[:3])


def check_quantize_scale_closed_form():
    one = _bits([[1.0] * 32])
    assert oracle.quantize(MXFP4, one, None, 1, 32)[1][0, 0] == 127 - 2     # 1 = 2^0, emax 2
    assert oracle.quantize(MXFP8, one, None, 1, 32)[1][0, 0] == 127 - 8     # emax 8
    six = _bits([[6.0] + [0.0] * 31])
    assert oracle.quantize(MXFP4, six, None, 1, 32)[1][0, 0] == 127         # 6 in [4, 8): 2^(2-2)
    assert oracle.quantize(MXFP4, six, None, 1, 32)[0][0, 0] == 0x07        # code of 6
    zero = _bits([[0.0] * 32])
    assert oracle.quantize(MXFP4, zero, None, 1, 32)[1][0, 0] == 0           # exponent clamped to -127
    tiny = _bits([[2.0 ** -133] + [0.0] * 31])                               # smallest bf16 subnormal
    assert oracle.quantize(MXFP8, tiny, None, 1, 32)[1][0, 0] == 0


def check_quantize_roundtrip(fmt, seed=17):
    """Blocks whose largest code is 4 or 6 (E2M1) / has exponent field 15 (E4M3): the
    dequantized bf16 weights quantize back to the same codes and scales."""
    rng = np.random.default_rng(seed)
    n, k = 24, 128
    codes, scales, _, _ = _rand_case(fmt, rng, n, k, 100, 150)
    if fmt == MXFP4:
        nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(n, k)
        nib[:, ::32] = rng.choice([6, 7, 14, 15], size=(n, k // 32))      # one +-4 or +-6 per block
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    else:
        codes[:, ::32] = rng.choice([0x78, 0x7B, 0x7E, 0xF8, 0xFE], size=(n, k // 32))
    w = oracle.dequant(fmt, codes, scales, None, n, k)
    xb = torch.from_numpy(w).to(torch.bfloat16)
    assert torch.equal(xb.float(), torch.from_numpy(w)), "decoded weights are bf16 values"
    x = xb.view(torch.int16).numpy().view(np.uint16)
    qc, qs = oracle.quantize(fmt, x, None, n, k)
    assert (qs == scales).all()
    assert (qc == codes).all()


# ---- FP8 block checkpoint -> MXFP8 ---------------------------------------------------------
# Independent reference: torch's E4M3 decoder, the tile scale applied by one numpy float32
# multiplication, then the MX steps of _quantize_reference on the fp32 values.

def _requant_reference(codes_in, tile_scales, n, k, bn, bk):
    q = torch.from_numpy(codes_in.copy()).view(torch.float8_e4m3fn).float().numpy()
    tr, tc = np.arange(n)[:, None] // bn, np.arange(k)[None, :] // bk
    v = (q * tile_scales[tr, tc]).astype(np.float32)          # float32 product: one rounding
    e4m3 = _grid("e4m3")
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 32), dtype=np.uint8)
    for r in range(n):
        for b in range(k // 32):
            blk = v[r, b * 32:(b + 1) * 32].astype(np.float64)
            amax = float(np.max(np.abs(blk)))
            se = -127 if amax == 0 else min(127, max(-127, math.frexp(amax)[1] - 1 - 8))
            scales[r, b] = se + 127
            for j, val in enumerate(blk):
                neg = 1 if np.signbit(val) else 0
                codes[r, b * 32 + j] = _nearest(abs(val) / 2.0 ** se, e4m3) | (neg << 7)
    return codes, scales


def _finite_e4m3(rng, shape, lo=0, hi=15):
    """Random E4M3 bytes with exponent field in [lo, hi], any sign and mantissa, never NaN."""
    pool = np.array([c for c in range(256) if lo <= (c >> 3) & 15 <= hi and (c & 0x7F) != 0x7F], dtype=np.uint8)
    return pool[rng.integers(0, pool.size, size=shape)]


def _requant_tie_case(count=24):
    """Blocks where the fp32 rounding of the dequantized value decides the E4M3 code:
    q * s (exact) lies just above a midpoint m of two E4M3 values whose lower one has the
    even code, and fl32(q * s) == m, which then rounds down (ties to even) while the
    exact product rounds up.  Each 32-block: 256 (sets the MX scale to 2^0 for s in
    [1, 2)) and 31 copies of q, with its own tile scale s (bn = 1, bk = 32)."""
    from fractions import Fraction as Fr
    grid = sorted((v, c) for v, c in _grid("e4m3") if v > 0)
    rows = []
    for (lo, clo), (hi, _) in zip(grid, grid[1:]):
        m = (lo + hi) / 2
        if clo % 2 or not 1.0 <= m <= 400.0:
            continue
        for q, cq in grid:
            if q < 1.0 or not 1 <= Fr(m) / Fr(q) < 2:
                continue
            s32 = np.float32(float(Fr(m) / Fr(q)))
            if Fr(float(s32)) <= Fr(m) / Fr(q):
                s32 = np.nextafter(s32, np.float32(2))
            exact = Fr(float(s32)) * Fr(q)
            if exact > Fr(m) and Fr(float(np.float32(float(exact)))) == Fr(m):
                rows.append((float(s32), cq))
                break
        if len(rows) >= count:
            break
    assert len(rows) >= 8
    codes = np.array([[0x78] + [cq] * 31 for _, cq in rows], dtype=np.uint8)
    ts = np.array([[s] for s, _ in rows], dtype=np.float32)
    return codes, ts


def check_requant_nearest(seed=23):
    rng = np.random.default_rng(seed)
    codes, ts = _requant_tie_case()
    n = codes.shape[0]
    c, sc = oracle.requant_fp8(codes, ts, n, 32, 1, 32)
    rc, rs = _requant_reference(codes, ts, n, 32, 1, 32)
    assert (sc == rs).all() and (c == rc).all(), "fp32 rounding of the dequantized values"
    for n, k, bn, bk in ((70, 288, 32, 128), (40, 96, 64, 32), (3, 32, 1, 32)):
        codes = _finite_e4m3(rng, (n, k))
        tiles = (-(-n // bn), -(-k // bk))
        ts = (rng.standard_normal(tiles) * np.exp2(rng.integers(-30, 30, size=tiles))).astype(np.float32)
        ts.flat[0] = np.float32(2.0 ** -7)                       # a power of two among them
        codes[0, :32] = 0x80                                     # a block of negative zeros
        codes[1, :32] = _finite_e4m3(rng, 32, 0, 0)              # a block of E4M3 subnormals
        c, sc = oracle.requant_fp8(codes, ts, n, k, bn, bk)
        rc, rs = _requant_reference(codes, ts, n, k, bn, bk)
        assert (sc == rs).all(), (n, k, bn, bk, np.argwhere(sc != rs)[:3])
        assert (c == rc).all(), (n, k, bn, bk, np.argwhere(c != rc)[:3])


def check_requant_roundtrip(seed=29):
    """Tile scales 2^t (a different t per tile) and every 32-block holding a value of
    exponent field 15 and only normal values: the MX scale is exactly the tile scale
    (byte t + 127) and the codes come back unchanged."""
    rng = np.random.default_rng(seed)
    n, k, bn, bk = 96, 384, 64, 128
    codes = _finite_e4m3(rng, (n, k), 1, 15)
    codes[:, ::32] = rng.choice([0x78, 0x7A, 0x7E, 0xF9, 0xFE], size=(n, k // 32))   # 256 .. 448, either sign
    t = rng.integers(-20, 10, size=(2, 3))
    ts = np.exp2(t).astype(np.float32)
    c, sc = oracle.requant_fp8(codes, ts, n, k, bn, bk)
    assert (c == codes).all()
    want = (t[np.arange(n)[:, None] // bn, (np.arange(k // 32)[None, :] * 32) // bk] + 127)
    assert (sc == want).all()


# ---- two-term E4M3 split of bf16 activations ------------------------------------------

def _e4m3_book():
    """Positive finite E4M3 codes 0x00 .. 0x7E and their values (decoded by the pinned oracle.e4m3)."""
    codes = np.arange(0x7F)
    return codes, np.array([oracle.e4m3(int(c)) for c in codes])


def _split_bruteforce(v):
    """Brute-force split of fp64 blocks v [nblocks][32]: each scale exponent found by searching
    e = -127 .. 127 for the smallest with amax <= 448 * 2^e, each code by searching the E4M3
    codebook for the nearest value (ties: the even code).  Returns (q1, q2, e1, e2) like
    oracle.split_e4m3 (codes with sign bits, E8M0 bytes)."""
    book_c, book_v = _e4m3_book()
    es = np.arange(-127, 128)

    def exponent(amax):
        ok = amax[:, None] <= 448.0 * np.exp2(es)[None, :]
        return np.where(ok.any(axis=1), es[np.argmax(ok, axis=1)], 127)

    def nearest(t):  # t >= 0, fp64 -> index into the codebook (searched once per distinct value)
        u, inv = np.unique(t, return_inverse=True)
        d = np.abs(book_v[None, :] - u[:, None])
        cand = d == d.min(axis=1, keepdims=True)
        even = cand & (book_c[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
        return pick[inv.reshape(-1)].reshape(t.shape)

    neg1 = np.signbit(v)
    e1 = exponent(np.abs(v).max(axis=1))
    i1 = nearest(np.abs(v) / np.exp2(e1)[:, None])
    m1 = book_v[i1]
    r = v - np.where(neg1, -m1, m1) * np.exp2(e1)[:, None]
    e2 = exponent(np.abs(r).max(axis=1))
    i2 = nearest(np.abs(r) / np.exp2(e2)[:, None])
    q1 = (book_c[i1] | (neg1.astype(np.int64) << 7)).astype(np.uint8)
    q2 = (book_c[i2] | ((r < 0).astype(np.int64) << 7)).astype(np.uint8)
    return q1, q2, (e1 + 127).astype(np.uint8), (e2 + 127).astype(np.uint8)


def _split_check(xbits):
    rows, k = xbits.shape
    got = oracle.split_e4m3(xbits, rows, k)
    v = (xbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 32)
    want = _split_bruteforce(v)
    for name, g, w in zip(("q1", "q2", "e1", "e2"), got, want):
        g = g.reshape(w.shape)
        assert (g == w).all(), (name, np.argwhere(g != w)[:3], g[g != w][:3], w[g != w][:3])


def check_split_every_bf16():
    """Every finite bf16 value alone in a block (the other 31 elements zero, both signs of zero)."""
    h = np.arange(65536, dtype=np.uint32)
    finite = ((h >> 7) & 0xFF) != 0xFF
    vals = h[finite].astype(np.uint16)
    x = np.zeros((vals.size, 32), dtype=np.uint16)
    x[:, 0] = vals
    x[:, 17] = 0x8000  # -0 keeps its sign in term 1
    _split_check(x)


def check_split_mixed_blocks(seed=47):
    """Blocks mixing magnitudes over many binades, subnormals, zeros and values near the bf16 top;
    and the exactness the design relies on: N(0,1) activations are reproduced exactly by the two
    terms for all but a small fraction of elements."""
    rng = np.random.default_rng(seed)
    rows = [(rng.standard_normal(64) * np.exp2(rng.integers(-30, 30, size=64))).tolist() for _ in range(8)]
    rows.append([1e-39, -2e-40] + [0.0] * 62)
    rows.append([3.0e38, -1.0] + [7.0] * 62)
    rows.append([448.0, 449.0, 447.0, -0.0] * 16)
    _split_check(_bits(rows))
    x = _bits(rng.standard_normal((64, 256)).tolist())
    q1, q2, e1, e2 = oracle.split_e4m3(x, 64, 256)
    dec = np.vectorize(oracle.e4m3)
    s1 = np.repeat(np.exp2(e1.astype(np.float64) - 127), 32, axis=1)
    s2 = np.repeat(np.exp2(e2.astype(np.float64) - 127), 32, axis=1)
    v = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert (dec(q1) * s1 + dec(q2) * s2 == v).mean() > 0.999


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
                (f"gemm_rows_{f}", lambda f=f: check_gemm_rows_bruteforce(f)),
                (f"moe_block_{f}", lambda f=f: check_moe_block(f))]
    out += [("route", check_route), ("silu", check_silu), ("round_bf16", check_round_bf16),
            ("swiglu_tie", check_swiglu_tie), ("block_rounding_bound", check_block_rounding_bound),
            ("block_rounding_bound_bruteforce", check_block_rounding_bound_bruteforce)]
    out += [(f"quantize_nearest_{f}", lambda f=f: check_quantize_nearest(f)) for f in FMTS]
    out += [("quantize_scale_closed_form", check_quantize_scale_closed_form),
            ("quantize_roundtrip_mxfp4", lambda: check_quantize_roundtrip(MXFP4)),
            ("quantize_roundtrip_mxfp8", lambda: check_quantize_roundtrip(MXFP8)),
            ("requant_nearest", check_requant_nearest), ("requant_roundtrip", check_requant_roundtrip)]
    out += [("split_every_bf16", check_split_every_bf16), ("split_mixed_blocks", check_split_mixed_blocks)]
    return out
