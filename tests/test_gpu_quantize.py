"""Block-float quantizer parity: codes and block scales written by the HIP
kernel equal the CPU oracle's bit for bit (a quantized code is a decision, so
both sides take it on the same fp32 values)."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import oracle_pins as pins
import synth
from gpu_util import dev_bf16, dev_f32, host, say

pytestmark = pytest.mark.gpu

FMT_NAMES = {1: "mxfp4", 2: "mxfp8", 3: "nvfp4"}


def bf16_spread(rng, rows, k, lo=-20, hi=20):
    """bf16 values N(0,1) times 2^U[lo, hi): many binades, both signs."""
    f = (rng.standard_normal((rows, k)) * np.exp2(rng.integers(lo, hi, size=(rows, k)))).astype(np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def check(fmt, x, g, what):
    say(what)
    rows, k = x.shape
    gd = None if g is None else dev_f32(np.array([g], dtype=np.float32))
    codes, scales = mxq.quantize(fmt, dev_bf16(x), gd)
    codes, scales = host(codes), host(scales)
    rc, rs = oracle.quantize(fmt, x, g, rows, k)
    bad_s = np.argwhere(scales != rs)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale bytes differ, first {bad_s[0]}"
    bad_c = np.argwhere(codes != rc)
    assert bad_c.size == 0, f"{what}: {len(bad_c)} code bytes differ, first {bad_c[0]}"


NV_G = [float(np.float32(1.0 / 2688.0)), 0.75, float(np.float32(3.0e-3))]


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("rows,k", [(37, 1024), (5, 96), (300, 32), (1, 4096)])
def test_random_matches_oracle(fmt, rows, k):
    rng = np.random.default_rng(rows * 7 + k + fmt)
    x = bf16_spread(rng, rows, k)
    for g in (NV_G if fmt == 3 else [None]):
        check(fmt, x, g, f"quantize {FMT_NAMES[fmt]} {rows}x{k} g={g}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_special_blocks_match_oracle(fmt):
    """Exact ties of the element grids, zero blocks, -0, bf16 subnormals (scale
    clamp), values near the top of bf16 (NVFP4 quotients that overflow)."""
    x = pins._quant_cases(fmt, 70 + fmt)
    for g in (NV_G if fmt == 3 else [None]):
        check(fmt, x, g, f"quantize special {FMT_NAMES[fmt]} g={g}")


@pytest.mark.parametrize("g", [2.0 ** -60, 1e-30, 1.0, 2.0 ** 60, 3.0e5])
def test_nvfp4_quotients_over_the_whole_exponent_range(g):
    """NVFP4 element quotients v / fl32(s g) with v over bf16's whole exponent
    range and global scales that put fl32(s g) far from 1: every path of the
    quotient (one reciprocal per block plus a residual step, and the plain
    division for operands and scales far from 1) against the oracle's
    division, bit for bit."""
    rng = np.random.default_rng(int(np.log2(g) + 200) if g > 0 else 1)
    x = bf16_spread(rng, 96, 512, -125, 126)
    x[::7] = bf16_spread(rng, 14, 512, -3, 3)  # every 7th row: one narrow range, quotients near the grid
    check(3, x, float(np.float32(g)), f"quantize nvfp4 wide exponents g={g}")


@pytest.mark.parametrize("fmt", [1, 2])
def test_roundtrip_through_device_decode(fmt):
    """Weights whose blocks peak at the format's top binade: GPU dequant -> bf16 ->
    GPU quantize gives back the original codes and scales."""
    sc, ss, _, _, _ = synth.streams(80 + fmt)
    n, k = 96, 512
    codes, scales, _ = synth.weights(fmt, sc, ss, n, k, 100, 150)
    if fmt == 1:
        nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(n, k)
        nib[:, ::32] = 7
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    else:
        codes[:, ::32] = 0x7E
    say("quantize round trip", fmt)
    w = mxq.dequant(fmt, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    xb = w.to(torch.bfloat16)
    assert torch.equal(xb.float(), w)
    qc, qs = mxq.quantize(fmt, xb)
    assert (host(qs) == scales).all()
    assert (host(qc) == codes).all()


def test_full_size_gate_up_sampled():
    """A 51200 x 5120 bf16 N(0,1) matrix (the gate/up shape) to MXFP4; the oracle
    checks 256 seeded rows in full."""
    rng = np.random.default_rng(90)
    rows, k = 51200, 5120
    say("quantize 51200x5120 mxfp4")
    xt = torch.randn(rows, k, generator=torch.Generator().manual_seed(90)).to(torch.bfloat16)
    codes, scales = mxq.quantize(1, xt.cuda())
    pick = np.sort(rng.choice(rows, 256, replace=False))
    xs = xt[pick].view(torch.int16).numpy().view(np.uint16)
    rc, rs = oracle.quantize(1, xs, None, len(pick), k)
    assert (host(scales)[pick] == rs).all()
    assert (host(codes)[pick] == rc).all()
