"""In-kernel decode, bit for bit: mxq_dequant (the scaled-conversion decode the
GEMV, MoE and GEMM kernels run, with the same MXFP8 lift for E8M0 bytes below
3) against the oracle's fp32 decode, over every code x every scale byte of each
format, including subnormal, overflow and NaN scales.  The product kernels
themselves are checked through one-hot activations in test_gpu_decode_paths."""
import numpy as np
import pytest

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import dev_f32, dev_u8, host, same_bits_f32, say
from oracle_pins import exhaustive_tile

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,g", [(1, None), (2, None), (3, 1.0), (3, 0.125), (3, float(np.float32(1 / 2688)))])
def test_exhaustive_decode_tile(fmt, g):
    codes, scales, gg, rows, k = exhaustive_tile(fmt, g)
    say("dequant exhaustive", fmt, g)
    w = host(mxq.dequant(fmt, dev_u8(codes), dev_u8(scales), dev_f32(gg)))
    ref = oracle.dequant(fmt, codes, scales, gg, rows, k)
    ok = same_bits_f32(w, ref)
    assert ok.all(), (np.argwhere(~ok)[:5], w[~ok][:5], ref[~ok][:5])


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("rows,k", [(3, 32), (37, 1024), (5, 5120)])
def test_random_decode(fmt, rows, k):
    sc, ss, _, _, _ = synth.streams(fmt * 100 + rows)
    codes, scales, g = synth.weights(fmt, sc, ss, rows, k, 0, 254)
    say("dequant random", fmt, rows, k)
    w = host(mxq.dequant(fmt, dev_u8(codes), dev_u8(scales), dev_f32(g)))
    ref = oracle.dequant(fmt, codes, scales, g, rows, k)
    assert same_bits_f32(w, ref).all()


def test_nvfp4_half_chunk_rows():
    """NVFP4 rows of k = 48 (24 code bytes) take the 8-byte chunk path."""
    sc, ss, _, _, _ = synth.streams(9)
    codes, scales, g = synth.weights(3, sc, ss, 7, 48)
    say("dequant nvfp4 k=48")
    w = host(mxq.dequant(3, dev_u8(codes), dev_u8(scales), dev_f32(g)))
    assert same_bits_f32(w, oracle.dequant(3, codes, scales, g, 7, 48)).all()
