"""Prefill GEMM parity: fp32 output against the oracle (every output at small
sizes, 64 seeded token rows at the full 4096 x 25600 x 5120 size), the bf16
output equal to round-to-nearest-even of the fp32 output, and GEMM rows equal
to the GEMV of the same token."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import assert_within, dev_bf16, dev_f32, dev_u8, host, say

pytestmark = pytest.mark.gpu


def small_case(fmt, m, n, k, seed):
    sc, ss, sx, _, _ = synth.streams(seed)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k, 120, 130)
    X = synth.bf16_normal(sx, (m, k))
    return dict(fmt=fmt, codes=codes, scales=scales, g=g, x=X, m=m, n=n, k=k)


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("m,n,k", [(300, 200, 256), (128, 128, 64), (1, 7, 32), (257, 129, 96), (2, 300, 5120),
                                   (5, 77, 256), (9, 129, 96), (16, 1000, 512), (17, 200, 256), (32, 64, 128),
                                   (33, 96, 64)])
def test_gemm_all_outputs(fmt, m, n, k):
    c = small_case(fmt, m, n, k, m + n + k + fmt)
    say("gemm", fmt, m, n, k)
    Y = host(mxq.gemm(fmt, dev_u8(c["codes"]), dev_u8(c["scales"]), dev_bf16(c["x"]), dev_f32(c["g"]),
                      out_dtype=torch.float32))
    Y_ref, A_ref = oracle.gemm_rows(fmt, c["codes"], c["scales"], c["g"], c["x"], np.arange(m), n, k)
    assert_within(Y, Y_ref, A_ref, f"gemm fmt={fmt} {m}x{n}x{k}")


@pytest.mark.parametrize("fmt", [1, 3])
@pytest.mark.parametrize("m", [260, 3, 16, 29])
def test_bf16_output_is_rne_of_fp32(fmt, m):
    """Both paths: 256 x 256 tiles (m > 32) and the matrix-unit GEMV (m <= 32, 16 rows a launch)."""
    c = small_case(fmt, m, 300, 512, 11)
    args = (fmt, dev_u8(c["codes"]), dev_u8(c["scales"]), dev_bf16(c["x"]), dev_f32(c["g"]))
    say("gemm bf16 epilogue", fmt)
    y32 = mxq.gemm(*args, out_dtype=torch.float32)
    y16 = mxq.gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rne = y32.cpu().to(torch.bfloat16)
    assert torch.equal(y16.cpu().view(torch.int16), rne.view(torch.int16))


@pytest.mark.parametrize("m,n,k", [(1, 7, 16), (40, 200, 48), (300, 129, 80), (17, 64, 1040), (260, 300, 5136)])
def test_nvfp4_rows_of_an_odd_number_of_blocks(m, n, k):
    """NVFP4 with k an odd multiple of 16: 8-byte rows whose last 32-element fragment
    holds one block (the matrix-unit GEMV needs whole 32-element blocks, so every m
    runs on the tiles); every output, and bf16 = RNE(fp32)."""
    c = small_case(3, m, n, k, m + n + k)
    say("gemm nvfp4 half-block rows", m, n, k)
    args = (3, dev_u8(c["codes"]), dev_u8(c["scales"]), dev_bf16(c["x"]), dev_f32(c["g"]))
    y32 = mxq.gemm(*args, out_dtype=torch.float32)
    y16 = mxq.gemm(*args, out_dtype=torch.bfloat16)
    Y_ref, A_ref = oracle.gemm_rows(3, c["codes"], c["scales"], c["g"], c["x"], np.arange(m), n, k)
    assert_within(host(y32), Y_ref, A_ref, f"gemm nvfp4 {m}x{n}x{k}")
    torch.cuda.synchronize()
    assert torch.equal(y16.cpu().view(torch.int16), y32.cpu().to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("fmt,k", [(1, 64), (2, 64), (3, 64), (3, 80)])
def test_last_round_in_smaller_tiles(fmt, k):
    """260 x 33357: 2 x 131 tiles of 256 x 256 leave a partly filled last round on
    a 256-CU device (one workgroup per CU), so the last 3 tile columns (589
    columns, ragged) run as a second launch of 128 x 128 tiles; NVFP4 also with
    8-byte rows (k = 80); every output."""
    m, n = 260, 33357
    c = small_case(fmt, m, n, k, 400 + fmt)
    say("gemm last round in smaller tiles", fmt)
    Y = host(mxq.gemm(fmt, dev_u8(c["codes"]), dev_u8(c["scales"]), dev_bf16(c["x"]), dev_f32(c["g"]),
                      out_dtype=torch.float32))
    Y_ref, A_ref = oracle.gemm_rows(fmt, c["codes"], c["scales"], c["g"], c["x"], np.arange(m), n, k)
    assert_within(Y, Y_ref, A_ref, f"gemm fmt={fmt} {m}x{n}x{k}")


def test_gemm_rows_match_gemv():
    c = small_case(1, 9, 640, 1024, 12)
    say("gemm row == gemv")
    Y = host(mxq.gemm(1, dev_u8(c["codes"]), dev_u8(c["scales"]), dev_bf16(c["x"]), out_dtype=torch.float32))
    yv = host(mxq.gemv(1, dev_u8(c["codes"]), dev_u8(c["scales"]), dev_bf16(c["x"][:8])))
    _, A = oracle.gemm_rows(1, c["codes"], c["scales"], None, c["x"], np.arange(8), c["n"], c["k"])
    assert_within(Y[:8], yv.astype(np.float64), 2 * A, "gemm vs gemv")


def test_prefill_full_size_64_rows():
    """4096 bf16 token rows x MXFP4 25600 x 5120; the oracle checks 64 seeded rows in full."""
    c = synth.prefill(seed=0)
    say("prefill 4096x25600x5120 fp32 + bf16")
    codes, scales, X = dev_u8(c["codes"]), dev_u8(c["scales"]), dev_bf16(c["x"])
    y32 = mxq.gemm(1, codes, scales, X, out_dtype=torch.float32)
    y16 = mxq.gemm(1, codes, scales, X, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = c["rows"]
    Y = y32[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    Y_ref, A_ref = oracle.gemm_rows(1, c["codes"], c["scales"], None, c["x"], rows, c["n"], c["k"])
    assert_within(Y, Y_ref, A_ref, "prefill 64 rows")
    sub32 = y32[:512].cpu()
    assert torch.equal(y16[:512].cpu().view(torch.int16), sub32.to(torch.bfloat16).view(torch.int16))
    assert bool(torch.isfinite(y32).all())
