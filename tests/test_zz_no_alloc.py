"""mxq_moe_block_noalloc (the MoE decode block with its workspace -- gate/up
outputs and activations -- in the library's static device array) against mxq_moe_block (caller workspace) and the
oracle: two calls in a row, the second smaller, so the second call runs on the
array the first one left behind."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, dev_i32, dev_u8, host, say
from oracle_pins import ROUNDING_TOL_EXACT

pytestmark = pytest.mark.gpu


def _block(c, noalloc):
    gc, gs, gg = c["gu"]
    dc, ds, dg = c["dn"]
    y = mxq.moe_block(c["fmt"], dev_u8(gc), dev_u8(gs), dev_u8(dc), dev_u8(ds), dev_i32(c["ids"]), dev_f32(c["w"]),
                      dev_bf16(c["x"]), gu_global_scale=dev_f32(gg), dn_global_scale=dev_f32(dg), noalloc=noalloc)
    return host(y)


def _check(c, what):
    say(what, "(allocation-free entry point, then the workspace one)")
    y_na = _block(c, True)
    y_ws = _block(c, False)
    same = (y_na.view(np.uint32) == y_ws.view(np.uint32)) | (np.isnan(y_na) & np.isnan(y_ws))
    assert same.all(), f"{what}: {int((~same).sum())} outputs differ from mxq_moe_block"
    y_ref, a_ref, amb = oracle.moe_block(c["fmt"], *c["gu"], *c["dn"], c["ids"], c["w"], c["x"], c["experts"],
                                         c["hidden"], c["dff"], rounding_tol=ROUNDING_TOL_EXACT)
    ok = np.abs(y_na - y_ref) <= 1e-5 * a_ref + amb + 1e-6
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs outside the oracle's bound"


def test_noalloc_block_two_calls_second_smaller():
    # first call: 8 tokens of the 30B-A3B-like block (workspace 8 x 8 x 768 x 10 bytes)
    _check(synth.moe_block(8, seed=41, exact=True), "noalloc block T=8 H=2048 dff=768 top-8")
    # second call: fewer tokens, narrower experts (workspace 2 x 4 x 256 x 10 bytes)
    _check(synth.moe_block(2, seed=42, experts=16, hidden=512, dff=256, topk=4, exact=True),
           "noalloc block T=2 H=512 dff=256 top-4")


def test_noalloc_block_rejects_oversized_activations():
    """The LDS limit of the down kernel is checked before anything runs."""
    c = synth.moe_block(1, seed=43, experts=16, hidden=64, dff=4096, topk=16)
    with pytest.raises(mxq.MxqError) as e:
        _block(c, True)
    assert e.value.status == 5
