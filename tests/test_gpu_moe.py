"""Expert-indexed MoE GEMV parity against the oracle, plus MoE == dense GEMV on
the gathered expert, invalid ids -> NaN rows, and repeated ids."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import assert_within, dev_bf16, dev_f32, dev_i32, dev_u8, host, say

pytestmark = pytest.mark.gpu


def run(case, ids=None):
    ids = case["ids"] if ids is None else ids
    return host(mxq.moe_gemv(case["fmt"], dev_u8(case["codes"]), dev_u8(case["scales"]), dev_i32(ids),
                             dev_bf16(case["x"]), case["x_per_slot"], dev_f32(case["g"])))


def check(case, what, ids=None):
    ids = case["ids"] if ids is None else ids
    say(what)
    y = run(case, ids)
    y_ref, a_ref = oracle.moe_gemv(case["fmt"], case["codes"], case["scales"], case["g"], ids, case["x"],
                                   case["x_per_slot"], case["experts"], case["n"], case["k"])
    assert_within(y, y_ref, a_ref, what)
    return y


@pytest.mark.parametrize("which", ["gate_up", "down"])
@pytest.mark.parametrize("tokens", [1, 2, 3, 4, 5, 8])
def test_moe_layer_all_outputs(which, tokens):
    """128 experts, top-8 distinct ids per token; every routed output row checked."""
    case = synth.moe_layer(which, tokens, seed=0)
    check(case, f"moe {which} T={tokens}")


@pytest.mark.parametrize("fmt", [2, 3])
@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_moe_other_formats(fmt, which):
    case = synth.moe_layer(which, 2, seed=1, fmt=fmt, experts=16)
    check(case, f"moe fmt={fmt} {which}")


def test_moe_equals_dense_on_gathered_expert():
    case = synth.moe_layer("gate_up", 4, seed=2, experts=32)
    say("moe == dense")
    y = run(case)
    for t in range(case["tokens"]):
        for s in range(case["topk"]):
            e = case["ids"][t, s]
            yd = host(mxq.gemv(1, dev_u8(case["codes"][e]), dev_u8(case["scales"][e]), dev_bf16(case["x"][t:t + 1])))
            _, a_ref = oracle.gemv(1, case["codes"][e], case["scales"][e], None, case["x"][t:t + 1], case["n"], case["k"])
            assert_within(yd[0], y[t, s].astype(np.float64), 2 * a_ref[0], f"moe==dense t={t} s={s}")


def test_invalid_and_repeated_ids():
    case = synth.moe_layer("down", 3, seed=3, experts=8, topk=4)
    ids = np.array([[0, 7, -1, 3], [3, 3, 8, 0], [5, 5, 5, 5]], dtype=np.int32)
    y = check(case, "moe invalid/repeated ids", ids)
    assert np.isnan(y[0, 2]).all() and np.isnan(y[1, 2]).all()
    assert np.isfinite(y[0, 0]).all() and np.isfinite(y[2]).all()


def test_more_pairs_than_one_batch():
    """Nine pairs on one expert: the kernel takes them in two batches."""
    case = synth.moe_layer("gate_up", 8, seed=4, experts=4, topk=2)
    ids = np.zeros((8, 2), dtype=np.int32)
    ids[:, 1] = np.arange(8) % 4
    check(case, "moe 9+ pairs on expert 0", ids)


def test_many_rounds_on_one_expert():
    """Two tokens (two pairs per round), all sixteen slots on one expert: eight rounds."""
    sc, ss, sx, _, _ = synth.streams(66)
    codes, scales, g = synth.weights(1, sc, ss, 64, 768, experts=4)
    ids = np.full((2, 8), 3, dtype=np.int32)
    x = synth.bf16_normal(sx, (2, 8, 768))
    check(dict(fmt=1, codes=codes, scales=scales, g=g, ids=ids, x=x, x_per_slot=1, experts=4, n=64, k=768,
               tokens=2, topk=8), "moe 16 pairs on expert 3, rounds of 2")


def test_moe_activations_from_global_memory():
    """Eight activation vectors of 8192 elements do not fit the LDS budget: the
    kernel reads them from global memory."""
    sc, ss, sx, si, _ = synth.streams(77)
    codes, scales, g = synth.weights(1, sc, ss, 20, 8192, experts=4)
    ids = synth.moe_ids(si, 5, 2, 4)
    x = synth.bf16_normal(sx, (5, 2, 8192))
    check(dict(fmt=1, codes=codes, scales=scales, g=g, ids=ids, x=x, x_per_slot=1, experts=4, n=20, k=8192,
               tokens=5, topk=2), "moe k=8192 tokens=5 (x from global memory)")


@pytest.mark.parametrize("n,k", [(33, 64), (100, 96), (5, 4096)])
def test_moe_ragged_shapes(n, k):
    sc, ss, sx, si, _ = synth.streams(n + k)
    codes, scales, g = synth.weights(1, sc, ss, n, k, experts=6)
    ids = synth.moe_ids(si, 3, 2, 6)
    x = synth.bf16_normal(sx, (3, 2, k))
    check(dict(fmt=1, codes=codes, scales=scales, g=g, ids=ids, x=x, x_per_slot=1, experts=6, n=n, k=k,
               tokens=3, topk=2), f"moe ragged n={n} k={k}")


def test_moe_deterministic():
    case = synth.moe_layer("gate_up", 4, seed=5)
    say("moe determinism")
    y1 = run(case)
    assert (run(case).view(np.uint32) == y1.view(np.uint32)).all()
