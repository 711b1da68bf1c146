"""FP8 block checkpoint -> MXFP8 on the GPU (mxq_requant_fp8) against the oracle,
bit for bit: E8M0 scale bytes and E4M3 codes, on random checkpoints with partial
tiles and unequal tile sides, on blocks where the fp32 rounding of the dequantized
value decides the code, on exact round trips, and on a 7168 x 2048 weight with
128 x 128 tiles (the vendor layout)."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
from gpu_util import dev_u8, host, say
from oracle_pins import _finite_e4m3, _requant_tie_case

pytestmark = pytest.mark.gpu


def run(codes_in, ts, bn, bk):
    c, s = mxq.requant_fp8(dev_u8(codes_in), torch.from_numpy(np.ascontiguousarray(ts)).to("cuda:0"), bn, bk)
    return host(c), host(s)


def check(codes_in, ts, bn, bk, what):
    n, k = codes_in.shape
    say("requant", what, n, k, bn, bk)
    c, s = run(codes_in, ts, bn, bk)
    rc, rs = oracle.requant_fp8(codes_in, ts, n, k, bn, bk)
    assert (s == rs).all(), (what, np.argwhere(s != rs)[:4])
    assert (c == rc).all(), (what, np.argwhere(c != rc)[:4], c[c != rc][:4], rc[c != rc][:4])


@pytest.mark.parametrize("n,k,bn,bk", [(70, 288, 32, 128), (40, 96, 64, 32), (3, 32, 1, 32), (257, 1056, 128, 128),
                                       (129, 640, 128, 64)])
def test_random_checkpoints(n, k, bn, bk):
    rng = np.random.default_rng(n * k + bn)
    codes = _finite_e4m3(rng, (n, k))
    tiles = (-(-n // bn), -(-k // bk))
    ts = (rng.standard_normal(tiles) * np.exp2(rng.integers(-40, 40, size=tiles))).astype(np.float32)
    codes[0, :32] = 0x80                            # negative zeros
    codes[min(1, n - 1), :32] = _finite_e4m3(rng, 32, 0, 0)  # E4M3 subnormals
    check(codes, ts, bn, bk, "random")


def test_fp32_rounding_decides_the_code():
    codes, ts = _requant_tie_case()
    check(codes, ts, 1, 32, "ties")


def test_exact_round_trip():
    rng = np.random.default_rng(29)
    n, k, bn, bk = 96, 384, 64, 128
    codes = _finite_e4m3(rng, (n, k), 1, 15)
    codes[:, ::32] = rng.choice([0x78, 0x7A, 0x7E, 0xF9, 0xFE], size=(n, k // 32))
    t = rng.integers(-20, 10, size=(2, 3))
    c, s = run(codes, np.exp2(t).astype(np.float32), bn, bk)
    assert (c == codes).all()
    assert (s == t[np.arange(n)[:, None] // bn, (np.arange(k // 32)[None, :] * 32) // bk] + 127).all()


def test_vendor_layout_128x128():
    """A 7168 x 2048 FP8 weight with 128 x 128 tiles (scales of the size real checkpoints carry)."""
    rng = np.random.default_rng(5)
    n, k = 7168, 2048
    codes = _finite_e4m3(rng, (n, k))
    ts = (np.abs(rng.standard_normal((n // 128, k // 128))) * 1e-3 + 1e-5).astype(np.float32)
    check(codes, ts, 128, 128, "vendor 128x128")
