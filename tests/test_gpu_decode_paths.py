"""The shipped decode, bit for bit, through every product kernel.

Each row of the probe tile holds one (scale byte, code) pair: every code of the
format against every scale byte (E8M0 0..255 for MX formats, E4M3 0x00..0xFF for
NVFP4 at three per-tensor scales), placed at one of eight probe columns; every
other code of the row is zero and every block of the row carries the same scale
byte.  With a one-hot activation x = e_j the GEMV sums one product w * 1 and
zeros, so each output must equal the decoded weight w[r][j] of the oracle
exactly, including subnormal results (E8M0 bytes 0, 1, 2), overflow to infinity
(bytes 253, 254) and NaN scales (byte 255, E4M3 0x7F / 0xFF).  The expected
value is the oracle's own one-hot product (fp64 sum), which is the decoded
weight itself wherever the row's other weights are finite, and NaN where one of
them is infinite or NaN (inf * 0).  The only difference allowed is the sign of
a zero: a sum of -0 and +0 terms is +0.

The kernels checked: the FMA GEMV at batch 1 (and forced at batch 4), the
matrix-mode GEMV at batches 2 and 4 (and forced at batch 1), the matrix-unit
GEMV at batch 8 (and forced at batch 1), the expert-indexed MoE GEMV (one pair per
round at one token, two from two tokens up), the prefill GEMM on its tile path
(m > 32), its last-round launch of 128 x 128 tiles and its small-m path, and
the expert-batched MoE GEMM.  The MoE decode
block's down projection runs the FMA GEMV's decode (the same streaming engine).
"""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
from gpu_util import dev_bf16, dev_f32, dev_i32, dev_u8, host, say

pytestmark = pytest.mark.gpu

K = 512
J = np.array([0, 1, 33, 94, 159, 255, 300, 511])  # probe columns: both nibbles, several blocks and chunks
BF16_ONE = 0x3F80
NAMES = {1: "mxfp4", 2: "mxfp8", 3: "nvfp4"}
CASES = [(1, None), (2, None), (3, 1.0), (3, 0.125), (3, float(np.float32(1 / 2688)))]


def probe_tile(fmt, g):
    """codes, scales, g array, rows, probe column of each row, scale byte and code of each row."""
    ncodes = 256 if fmt == 2 else 16
    rows = 256 * ncodes
    u = np.repeat(np.arange(256), ncodes)
    c = np.tile(np.arange(ncodes), 256)
    col = J[(c + u) % 8]
    if fmt == 2:
        codes = np.zeros((rows, K), dtype=np.uint8)
        codes[np.arange(rows), col] = c
    else:
        codes = np.zeros((rows, K // 2), dtype=np.uint8)
        codes[np.arange(rows), col // 2] = (c << (4 * (col % 2))).astype(np.uint8)
    bs = 16 if fmt == 3 else 32
    scales = np.repeat(u.astype(np.uint8)[:, None], K // bs, axis=1)
    gg = None if fmt != 3 else np.array([g], dtype=np.float32)
    return codes, scales, gg, rows, col, u, c


def one_hot(cols):
    x = np.zeros((len(cols), K), dtype=np.uint16)
    x[np.arange(len(cols)), cols] = BF16_ONE
    return x


def check(y, w_cols, tile, what):
    """y[b][r] against the oracle's one-hot product for batch entry b (fp64, exact here)."""
    y = np.asarray(y, dtype=np.float32)
    w = np.asarray(w_cols, dtype=np.float32)
    ok = (y == w) | (np.isnan(y) & np.isnan(w))
    if not ok.all():
        _, _, _, _, col, u, c = tile
        bad = np.argwhere(~ok)
        msg = [f"{what}: {bad.shape[0]} of {ok.size} outputs differ from the oracle"]
        for b, r in bad[:6]:
            msg.append(f"  entry {b} row {r} (scale byte {u[r]}, code {c[r]}, column {col[r]}): "
                       f"kernel {y[b, r]!r} oracle {w[b, r]!r}")
        raise AssertionError("\n".join(msg))


@pytest.fixture(scope="module", params=CASES, ids=lambda p: f"{NAMES[p[0]]}-g{p[1]}")
def tile(request):
    fmt, g = request.param
    t = probe_tile(fmt, g)
    codes, scales, gg, rows, _, _, _ = t
    w = oracle.dequant(fmt, codes, scales, gg, rows, K)
    # the one-hot products of the oracle at the eight probe columns, [8][rows]
    y_ref = oracle.gemv(fmt, codes, scales, gg, one_hot(J), rows, K)[0].astype(np.float32)
    # premise: wherever a row's weights are all finite the product is the decoded weight
    fin = np.isfinite(w).all(axis=1)
    assert (y_ref[:, fin] == w[fin][:, J].T).all()
    return dict(fmt=fmt, g=gg, t=t, w=w, y_ref=y_ref, rows=rows, host=(codes, scales, gg),
                codes=dev_u8(codes), scales=dev_u8(scales), gdev=dev_f32(gg))


def test_dequant(tile):
    """mxq_dequant against the oracle's decode, every element of the tile."""
    say("decode paths: dequant", NAMES[tile["fmt"]])
    w = host(mxq.dequant(tile["fmt"], tile["codes"], tile["scales"], tile["gdev"]))
    ref = tile["w"]
    ok = (w.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(w) & np.isnan(ref))
    assert ok.all(), (np.argwhere(~ok)[:5], w[~ok][:5], ref[~ok][:5])


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_gemv(tile, batch):
    """Batch 1: FMA rows; batches 2, 4: matrix-mode rows; batch 8: matrix-unit GEMV."""
    fmt = tile["fmt"]
    for b0 in range(0, 8, batch):
        cols = J[b0:b0 + batch]
        say("decode paths: gemv", NAMES[fmt], "batch", batch, "columns", list(cols))
        y = host(mxq.gemv(fmt, tile["codes"], tile["scales"], dev_bf16(one_hot(cols)), tile["gdev"]))
        check(y, tile["y_ref"][b0:b0 + batch], tile["t"], f"gemv batch {batch} columns {list(cols)}")


@pytest.mark.parametrize("path", [1, 2, 4])
def test_gemv_forced_paths(tile, path):
    """Batch 1 through the matrix-unit GEMV (1), batch 4 through the FMA rows (2), and
    batch 1 through the matrix-mode rows (4): the paths the default choice does not take
    at those batches."""
    fmt = tile["fmt"]
    batch = 4 if path == 2 else 1
    for b0 in range(0, 8, batch):
        cols = J[b0:b0 + batch]
        say("decode paths: gemv path", path, NAMES[fmt], list(cols))
        y = host(mxq.gemv(fmt, tile["codes"], tile["scales"], dev_bf16(one_hot(cols)), tile["gdev"],
                          config=dict(path=path)))
        check(y, tile["y_ref"][b0:b0 + batch], tile["t"], f"gemv path {path} columns {list(cols)}")


def _bank(tile):
    """Two experts: the tile and the tile with its rows reversed."""
    c = torch.stack([tile["codes"], tile["codes"].flip(0)]).contiguous()
    s = torch.stack([tile["scales"], tile["scales"].flip(0)]).contiguous()
    g = None if tile["g"] is None else dev_f32(np.repeat(tile["g"], 2))
    return c, s, g


def _moe_expect(tile, ids):
    """Pair (t, s) reads expert ids[t][s] (expert 1 = rows reversed) at probe column (t * topk + s) % 8."""
    y0 = tile["y_ref"]
    tokens, topk = ids.shape
    exp = np.empty((tokens, topk, tile["rows"]), dtype=np.float32)
    for t in range(tokens):
        for s in range(topk):
            y = y0[(t * topk + s) % 8]
            exp[t, s] = y if ids[t, s] == 0 else y[::-1]
    return exp


@pytest.mark.parametrize("tokens,topk", [(1, 8), (4, 2)])
def test_moe_gemv(tile, tokens, topk):
    fmt = tile["fmt"]
    c, s, g = _bank(tile)
    ids = np.array([[(t + q) % 2 for q in range(topk)] for t in range(tokens)], dtype=np.int32)
    x = one_hot(J[np.arange(tokens * topk) % 8]).reshape(tokens, topk, K)
    say("decode paths: moe gemv", NAMES[fmt], tokens, topk)
    y = host(mxq.moe_gemv(fmt, c, s, dev_i32(ids), dev_bf16(x), 1, g))
    exp = _moe_expect(tile, ids)
    check(y.reshape(-1, tile["rows"]), exp.reshape(-1, tile["rows"]), tile["t"], f"moe gemv T={tokens} topk={topk}")


@pytest.mark.parametrize("m", [64, 8])
def test_gemm(tile, m):
    """m = 64: the 256 x 256 MFMA tiles; m = 8: the small-m (matrix-unit GEMV) path."""
    fmt = tile["fmt"]
    cols = J[np.arange(m) % 8]
    say("decode paths: gemm", NAMES[fmt], "m", m)
    Y = host(mxq.gemm(fmt, tile["codes"], tile["scales"], dev_bf16(one_hot(cols)), tile["gdev"],
                      out_dtype=torch.float32))
    check(Y, tile["y_ref"][np.arange(m) % 8], tile["t"], f"gemm m={m}")


def test_gemm_last_round_tiles(tile):
    """The prefill GEMM's second launch, 128 x 128 tiles for a partly filled last
    round of 256 x 256 tiles: the probe rows (for MXFP8 those of scale bytes 0-3,
    127, 200, 254 and 255) sit after 65536 rows of zero weights, so a 64-row
    product has 256 + 16 (MXFP8: + 8) tile columns and, with one 256 x 256
    workgroup per CU on 256 CUs, the probe rows' columns are exactly the ones the
    second launch takes.  Each output against the oracle's one-hot product."""
    fmt = tile["fmt"]
    codes, scales, gg = tile["host"]
    t = tile["t"]
    sel = np.isin(t[5], [0, 1, 2, 3, 127, 200, 254, 255]) if fmt == 2 else np.ones(tile["rows"], dtype=bool)
    pad = 65536
    zc = np.zeros((pad, codes.shape[1]), dtype=np.uint8)
    zs = np.full((pad, scales.shape[1]), 0x38 if fmt == 3 else 127, dtype=np.uint8)  # unit scales
    C, S = np.vstack([zc, codes[sel]]), np.vstack([zs, scales[sel]])
    m = 64
    cols = J[np.arange(m) % 8]
    say("decode paths: gemm last round", NAMES[fmt])
    Y = host(mxq.gemm(fmt, dev_u8(C), dev_u8(S), dev_bf16(one_hot(cols)), tile["gdev"], out_dtype=torch.float32))
    assert (Y[:, :pad] == 0).all()
    t_sel = t[:4] + (t[4][sel], t[5][sel], t[6][sel])
    check(Y[:, pad:], tile["y_ref"][np.arange(m) % 8][:, sel], t_sel, "gemm last round")


def test_moe_gemm(tile):
    fmt = tile["fmt"]
    c, s, g = _bank(tile)
    tokens, topk = 4, 2
    ids = np.array([[(t + q) % 2 for q in range(topk)] for t in range(tokens)], dtype=np.int32)
    x = one_hot(J[np.arange(tokens * topk) % 8]).reshape(tokens, topk, K)
    say("decode paths: moe gemm", NAMES[fmt])
    y = host(mxq.moe_gemm(fmt, c, s, dev_i32(ids), dev_bf16(x), 1, g, out_dtype=torch.float32))
    exp = _moe_expect(tile, ids)
    check(y.reshape(-1, tile["rows"]), exp.reshape(-1, tile["rows"]), tile["t"], "moe gemm")
