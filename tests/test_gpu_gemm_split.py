"""The prefill GEMM on the block-scaled matrix instruction (mxq_gemm_split):
the activation split bit for bit against the oracle's (codes and scale bytes,
on normal rows, rows spanning many binades, zero and subnormal blocks, values
at 448 and the top of bf16), and Y against the oracle's exact product within
the acceptance bound 1e-5 * sum|w x| + 1e-6 -- every output at sizes spanning
several tiles with ragged edges and k slices of 32, 64 seeded rows at the full
4096 x 25600 x 5120 size -- with the bf16 output equal to the round-to-nearest
-even of the fp32 one."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import assert_within, dev_bf16, dev_u8, host, say

pytestmark = pytest.mark.gpu


def _bits(rows):
    return torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def split_inputs(seed, m, k):
    rng = np.random.default_rng(seed)
    x = synth.bf16_normal(synth.streams(seed)[2], (m, k))
    wide = _bits((rng.standard_normal((8, k)) * np.exp2(rng.integers(-40, 40, size=(8, k)))).tolist())
    special = np.zeros((6, k), dtype=np.uint16)
    special[0] = _bits([[1e-39, -2e-40] * (k // 2)])[0]             # bf16 subnormals only
    special[1, ::7] = _bits([[3.0e38] * len(range(0, k, 7))])[0]    # the top of bf16, zeros between
    special[2] = _bits([[448.0, 449.0, 447.0, -0.0] * (k // 4)])[0]
    special[3] = _bits([[-0.0] * k])[0]
    special[4] = _bits([[1.0 + 2 ** -7, -(1.0 + 2 ** -7)] * (k // 2)])[0]
    x[: 8] = wide
    x[8:14] = special
    return x


def run_split(codes, scales, x, out_dtype=torch.float32):
    m, k = x.shape
    ws = torch.full((mxq.gemm_split_workspace_bytes(m, k),), 0xA5, dtype=torch.uint8, device="cuda:0")
    y = mxq.gemm_split(dev_u8(codes), dev_u8(scales), dev_bf16(x), out_dtype=out_dtype, workspace=ws)
    return y, ws


@pytest.mark.parametrize("m,k", [(40, 1024), (16, 32), (300, 96)])
def test_split_is_the_oracles(m, k):
    x = split_inputs(m + k, m, k)
    sc, ss, _, _, _ = synth.streams(1)
    codes, scales, _ = synth.weights(1, sc, ss, 64, k, 120, 130)
    say("gemm split: activation split", m, k)
    _, ws = run_split(codes, scales, x)
    got = [host(v) for v in mxq.gemm_split_workspace_views(ws, m, k)]
    want = oracle.split_e4m3(x, m, k)
    for name, g, w in zip(("q1", "q2", "e1", "e2"), got, want):
        assert (g == w).all(), (name, np.argwhere(g != w)[:4], g[g != w][:4], w[g != w][:4])


@pytest.mark.parametrize("m,n,k", [(300, 520, 320), (257, 129, 96), (1, 7, 32), (17, 300, 1024), (512, 256, 64),
                                   (33, 1000, 352)])
def test_gemm_split_all_outputs(m, n, k):
    sc, ss, sx, _, _ = synth.streams(m + n + k)
    codes, scales, _ = synth.weights(1, sc, ss, n, k, 120, 130)
    x = synth.bf16_normal(sx, (m, k))
    say("gemm split", m, n, k)
    y32, _ = run_split(codes, scales, x, torch.float32)
    y16, _ = run_split(codes, scales, x, torch.bfloat16)
    Y_ref, A_ref = oracle.gemm_rows(1, codes, scales, None, x, np.arange(m), n, k)
    assert_within(host(y32), Y_ref, A_ref, f"gemm split {m}x{n}x{k}")
    torch.cuda.synchronize()
    assert torch.equal(y16.cpu().view(torch.int16), y32.cpu().to(torch.bfloat16).view(torch.int16))


def test_gemm_split_wide_activations():
    """Rows spanning many binades, subnormal and all-zero rows: still within the bound."""
    m, n, k = 64, 256, 512
    x = split_inputs(5, m, k)
    x[9] = 0  # the top-of-bf16 row is left out: its products overflow fp32 in any order
    sc, ss, _, _, _ = synth.streams(6)
    codes, scales, _ = synth.weights(1, sc, ss, n, k, 120, 130)
    say("gemm split wide activations")
    y, _ = run_split(codes, scales, x)
    Y_ref, A_ref = oracle.gemm_rows(1, codes, scales, None, x, np.arange(m), n, k)
    assert_within(host(y), Y_ref, A_ref, "gemm split wide activations")


def test_gemm_split_prefill_full_size_64_rows():
    """4096 bf16 token rows x MXFP4 25600 x 5120 (the prefill workload); 64 seeded rows in full."""
    c = synth.prefill(seed=0)
    say("gemm split prefill 4096x25600x5120")
    y, _ = run_split(c["codes"], c["scales"], c["x"])
    rows = c["rows"]
    Y_ref, A_ref = oracle.gemm_rows(1, c["codes"], c["scales"], None, c["x"], rows, c["n"], c["k"])
    assert_within(host(y)[rows], Y_ref, A_ref, "gemm split prefill rows")
