"""Expert-batched MoE GEMM parity: every routed (token, slot) pair's fp32 output
row against the CPU oracle (the expert-indexed product of each pair, fp64
sums), |y - y_ref| <= 1e-5 * sum|w x| + 1e-6; the bf16 output equal to
round-to-nearest-even of the fp32 output; rows equal to the expert-indexed
GEMV of the same token; NaN rows for ids outside the bank."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import assert_within, dev_bf16, dev_f32, dev_i32, dev_u8, host, say

pytestmark = pytest.mark.gpu

FMT_NAMES = {1: "mxfp4", 2: "mxfp8", 3: "nvfp4"}


def case(fmt, experts, n, k, m, topk, seed, per_slot=0, ids=None):
    sc, ss, sx, si, _ = synth.streams(seed)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k, experts=experts)
    if ids is None:
        ids = synth.moe_ids(si, m, topk, experts)
    x = synth.bf16_normal(sx, (m, topk, k) if per_slot else (m, k))
    return dict(fmt=fmt, codes=codes, scales=scales, g=g, ids=ids, x=x, per=per_slot, E=experts, n=n, k=k)


def run(c, out_dtype=torch.float32, ids=None):
    ids = c["ids"] if ids is None else ids
    y = mxq.moe_gemm(c["fmt"], dev_u8(c["codes"]), dev_u8(c["scales"]), dev_i32(ids), dev_bf16(c["x"]), c["per"],
                     global_scale=dev_f32(c["g"]), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def check(c, what, rows=None):
    say(what)
    y = host(run(c))
    ids, x = c["ids"], c["x"]
    if rows is not None:
        ids, x, y = ids[rows], x[rows], y[rows]
    y_ref, a_ref = oracle.moe_gemv(c["fmt"], c["codes"], c["scales"], c["g"], ids, x, c["per"], c["E"], c["n"],
                                   c["k"])
    assert_within(y, y_ref, a_ref, what)


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("E,n,k,m,topk,per", [(16, 200, 256, 37, 4, 0), (8, 300, 96, 130, 3, 0),
                                               (32, 129, 512, 20, 8, 1), (4, 64, 32, 1, 1, 0)])
def test_all_outputs(fmt, E, n, k, m, topk, per):
    """Several experts, ragged n tiles, every output of every pair checked."""
    c = case(fmt, E, n, k, m, topk, E + n + k + m + topk + fmt, per)
    check(c, f"moe gemm {FMT_NAMES[fmt]} E={E} n={n} k={k} m={m} topk={topk} per_slot={per}")


@pytest.mark.parametrize("E,n,k,m,topk,per", [(8, 100, 48, 30, 2, 0), (16, 129, 784, 40, 4, 1),
                                               (4, 64, 2064, 17, 2, 0)])
def test_nvfp4_rows_of_an_odd_number_of_blocks(E, n, k, m, topk, per):
    """NVFP4 with k an odd multiple of 16: the lane holding the last block holds half a
    block (8-byte code rows, one scale), every output checked."""
    c = case(3, E, n, k, m, topk, E + n + k + m, per)
    check(c, f"moe gemm nvfp4 half-block rows E={E} n={n} k={k} m={m} topk={topk} per_slot={per}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_one_expert_takes_several_row_tiles(fmt):
    """Every token routes to experts 0..3: expert 0 gets 600 pairs (three 256-row
    tiles, the last ragged), the other experts of the bank none."""
    m, topk = 600, 4
    ids = np.tile(np.arange(topk, dtype=np.int32), (m, 1))
    c = case(fmt, 8, 129, 128, m, topk, 77 + fmt, ids=ids)
    check(c, f"skewed routing {FMT_NAMES[fmt]}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("E,per", [(16, 0), (12, 1)])
def test_pair_scan_across_chunks(fmt, E, per):
    """4400 pairs: more than one 4096-pair scan chunk.  Slot 0 of most tokens
    routes to expert 0, so its ~900 pairs take 15 passes whose boundaries fall
    inside chunks and across the chunk boundary; 16 experts take the XCD-grouped
    workgroup order, 12 the plain one.  Every output checked."""
    m, topk = 1100, 4
    _, _, _, si, _ = synth.streams(150 + E + fmt)
    ids = synth.moe_ids(si, m, topk, E)
    rng = np.random.default_rng(E + fmt)
    for t in np.flatnonzero(rng.random(m) < 0.8):
        row = ids[t]
        if 0 in row:  # keep the token's experts distinct: swap expert 0 into slot 0
            row[np.flatnonzero(row == 0)[0]] = row[0]
        row[0] = 0
    c = case(fmt, E, 72, 96, m, topk, 160 + E + fmt, per, ids=ids)
    check(c, f"pair scan across chunks {FMT_NAMES[fmt]} E={E} per_slot={per}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_bf16_output_is_rne_of_fp32(fmt):
    c = case(fmt, 16, 300, 512, 70, 4, 90 + fmt)
    say("moe gemm bf16 epilogue", fmt)
    y32 = run(c, torch.float32)
    y16 = run(c, torch.bfloat16)
    rne = y32.cpu().to(torch.bfloat16)
    assert torch.equal(y16.cpu().view(torch.int16), rne.view(torch.int16))


def test_rows_match_expert_indexed_gemv():
    """The same pairs through the decode GEMV (mxq_moe_gemv): within twice the bound."""
    c = case(1, 32, 640, 1024, 8, 8, 101)
    say("moe gemm == moe gemv")
    y = host(run(c))
    yv = host(mxq.moe_gemv(1, dev_u8(c["codes"]), dev_u8(c["scales"]), dev_i32(c["ids"]), dev_bf16(c["x"]), 0))
    _, a_ref = oracle.moe_gemv(1, c["codes"], c["scales"], None, c["ids"], c["x"], 0, 32, 640, 1024)
    assert_within(y, yv.astype(np.float64), 2 * a_ref, "moe gemm vs moe gemv")


def test_invalid_ids_give_nan_rows():
    c = case(1, 16, 96, 256, 9, 4, 111)
    ids = c["ids"].copy()
    ids[2, 1] = 16
    ids[5, 3] = -1
    say("moe gemm invalid ids")
    for dt in (torch.float32, torch.bfloat16):
        y = run(c, dt, ids=ids).float().cpu().numpy()
        assert np.isnan(y[2, 1]).all() and np.isnan(y[5, 3]).all()
        ok = np.ones(ids.shape, dtype=bool)
        ok[2, 1] = ok[5, 3] = False
        assert np.isfinite(y[ok]).all()
    y = host(run(c, ids=ids))
    good = ids.copy()
    good[2, 1] = good[5, 3] = 0
    y_ref, a_ref = oracle.moe_gemv(1, c["codes"], c["scales"], None, good, c["x"], 0, 16, 96, 256)
    mask = np.ones(ids.shape, dtype=bool)
    mask[2, 1] = mask[5, 3] = False
    assert_within(y[mask], y_ref[mask], a_ref[mask], "valid pairs next to invalid ids")


def test_deterministic():
    c = case(1, 16, 384, 512, 200, 8, 121)
    say("moe gemm determinism")
    y1 = host(run(c))
    for _ in range(2):
        assert (host(run(c)).view(np.uint32) == y1.view(np.uint32)).all()


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_30b_a3b_prefill_sampled(fmt, which):
    """The 30B-A3B-like bank (128 experts; gate/up 1536 x 2048, down 2048 x 768,
    per-slot inputs) with 512 tokens x top-8 (a 512-token prompt); the oracle
    checks 24 seeded tokens (all 8 slots, every output) of the full launch."""
    n, k = synth.MOE_SHAPES[which]
    per = 1 if which == "down" else 0
    c = case(fmt, 128, n, k, 512, 8, (131 if per else 130) + 10 * (fmt - 1), per)
    rows = np.sort(np.random.default_rng(5).choice(512, 24, replace=False))
    check(c, f"30B-A3B {which} prefill {FMT_NAMES[fmt]}, 512 tokens", rows)


@pytest.mark.parametrize("per", [0, 1])
def test_mxfp8_lifted_blocks_among_others(per):
    """MXFP8 blocks with E8M0 bytes 0..2 (decoded 2^3 larger against inputs
    scaled by 2^-3) scattered among ordinary blocks, some rows holding both in
    one slice, next to blocks of large scales; every output checked."""
    c = case(2, 8, 96, 320, 40, 4, 180 + per, per)
    rng = np.random.default_rng(7 + per)
    sc = c["scales"].copy()
    pick = rng.random(sc.shape)
    sc[pick < 0.15] = rng.integers(0, 3, size=int((pick < 0.15).sum()))
    sc[(pick >= 0.15) & (pick < 0.2)] = 200
    c["scales"] = sc
    check(c, f"mxfp8 lifted blocks per_slot={per}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("k", [32, 96, 768, 1024, 1280, 2048, 2560, 3072, 4064, 4128, 7168, 16416])
def test_streaming_kernel_across_k(fmt, k):
    """Rows of whole 32-element blocks take the streaming kernel in every format:
    one slice or many, MXFP8's 32-wide slices and the others' 64-wide ones
    ending inside the last slice, and rows longer than the staging kernel's LDS
    allows (k > 4088); every output checked."""
    c = case(fmt, 8, 40, k, 21, 3, 140 + k + fmt)
    check(c, f"moe gemm streaming {FMT_NAMES[fmt]} k={k}")


@pytest.mark.parametrize("k", [16, 48, 80, 496, 752, 1008, 2032, 4080, 4112, 8208])
def test_nvfp4_8_byte_rows_across_k(k):
    """NVFP4 rows of an odd number of 16-element blocks (8-byte aligned rows):
    the streaming kernel loads each lane's share as two 8-byte halves and the
    row's last share holds one block; one slice or many, the last share in
    either half of its slice, rows past 4088; every output checked."""
    c = case(3, 8, 40, k, 21, 3, 170 + k)
    check(c, f"moe gemm nvfp4 8-byte rows k={k}")
