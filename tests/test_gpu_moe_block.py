"""MoE decode block on the GPU against the oracle: top-k softmax routing (ids
bit-exact, weights within fp32 rounding) and the fused block gate/up -> SwiGLU
-> down -> routing-weighted combine (the gate/up workspace and the outputs),
in every format, with odd topk, ragged sizes, invalid ids and repeated calls.

Tolerances:
  * routing weights: |w - w_ref| <= 1e-5 w_ref + 1e-7.  The kernel's fp32
    path is an exp per expert (a few ulp), a 64-lane tree sum of at most 1024
    positive terms (at most 22 roundings on any path), one division and, with
    renormalisation, a sum of at most 16 terms and one more division: well
    under 100 ulp = 6e-6 relative.
  * block outputs: |y - y_ref| <= 1e-5 abs_y + amb_y + 1e-6, where amb_y is the
    oracle's bound on what a legitimate choice of the other bf16 neighbour for
    an activation can move y (the rounding decision is taken on fp32 gate/up
    values whose last bits depend on the summation order).  With "exact"
    inputs every gate/up sum is an fp32 number in any order, so the gate/up
    workspace must match bit for bit and amb_y only covers the few activations
    within 8 fp32 ulp of a bf16 tie; with normal inputs the gate/up values
    carry the GEMV acceptance bound and amb_y is correspondingly wider.
"""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import assert_within, dev_bf16, dev_f32, dev_i32, dev_u8, host, say
from oracle_pins import ROUNDING_TOL_CONTRACT, ROUNDING_TOL_EXACT

pytestmark = pytest.mark.gpu


# ---- routing --------------------------------------------------------------------------

def route_case(seed, tokens, experts):
    rng = synth.streams(seed)[2]
    logits = synth.router_logits(rng, tokens, experts)
    # planted ties: two equal maxima in token 0; an all-equal row; a tie at
    # every selection boundary in the last token (pairs of equal values)
    logits[0, experts // 3] = logits[0, experts - 1] = logits[0].max() + np.float32(1.0)
    if tokens > 1:
        logits[1, :] = np.float32(0.25)
    if tokens > 2:
        logits[-1, 1::2] = logits[-1, 0::2][: experts // 2]
    return logits


@pytest.mark.parametrize("tokens,experts,topk", [(1, 128, 8), (4, 128, 8), (8, 128, 8), (3, 64, 6), (2, 6, 6),
                                                 (5, 1000, 16), (2, 1024, 1), (8, 200, 3), (3, 65, 5), (2, 300, 8),
                                                 (1, 512, 4)])
@pytest.mark.parametrize("renorm", [False, True])
def test_route(tokens, experts, topk, renorm):
    logits = route_case(tokens * 1000 + experts, tokens, experts)
    say(f"route T={tokens} E={experts} topk={topk} renorm={renorm}")
    ids, w = mxq.moe_route(dev_f32(logits), topk, renorm)
    ids, w = host(ids), host(w)
    ids_ref, w_ref = oracle.moe_route(logits, topk, renorm)
    assert (ids == ids_ref).all(), (np.argwhere(ids != ids_ref)[:4], ids, ids_ref)
    assert (np.abs(w - w_ref) <= 1e-5 * w_ref + 1e-7).all(), np.abs(w - w_ref).max()


def test_route_infinite_logits():
    logits = route_case(7, 2, 128)
    logits[0, 5] = -np.inf
    logits[1, :64] = -np.inf
    say("route with -inf logits")
    ids, w = mxq.moe_route(dev_f32(logits), 8, True)
    ids_ref, w_ref = oracle.moe_route(logits, 8, True)
    assert (host(ids) == ids_ref).all()
    assert (np.abs(host(w) - w_ref) <= 1e-5 * w_ref + 1e-7).all()


# ---- the block ------------------------------------------------------------------------

def run_block(c, ids=None, act=False):
    """y, the gate/up workspace h [T, topk, 2 dff] (and with act the bf16 activations as float32)."""
    ids = c["ids"] if ids is None else ids
    gc, gs, gg = c["gu"]
    dc, ds, dg = c["dn"]
    T, topk = ids.shape
    ws = torch.full((mxq.moe_block_workspace_elems(T, topk, c["dff"]),), float("nan"), dtype=torch.float32,
                    device="cuda:0")
    y = mxq.moe_block(c["fmt"], dev_u8(gc), dev_u8(gs), dev_u8(dc), dev_u8(ds), dev_i32(ids), dev_f32(c["w"]),
                      dev_bf16(c["x"]), gu_global_scale=dev_f32(gg), dn_global_scale=dev_f32(dg), h=ws)
    h, a = mxq.moe_block_workspace_views(ws, T, topk, c["dff"])
    return (host(y), host(h), host(a.float())) if act else (host(y), host(h))


def check_activations(h, a, what):
    """The activations the gate/up kernel wrote against the oracle's SwiGLU of the kernel's own gate/up values:
    bf16(fl32(fl32(silu(g)) * u)), either neighbour accepted where the fp32 product is within 8 fp32 ulp of a
    bf16 tie (the kernel's fp32 exp and division differ from the exact silu by a few ulp)."""
    dff = h.shape[-1] // 2
    g, u = h[..., :dff].reshape(-1), h[..., dff:].reshape(-1)
    a = a.reshape(-1)
    valid = np.isfinite(g) & np.isfinite(u)
    assert valid.any(), f"{what}: no finite gate/up values"
    bad = []
    for i in np.flatnonzero(valid):
        p = float(np.float32(np.float32(oracle.silu(float(g[i]))) * u[i]))
        lo, hi = oracle.round_bf16(p - abs(p) * 2.0 ** -21), oracle.round_bf16(p + abs(p) * 2.0 ** -21)
        if not (min(lo, hi) <= a[i] <= max(lo, hi)):
            bad.append((i, g[i], u[i], a[i], oracle.round_bf16(p)))
    assert not bad, f"{what}: {len(bad)} activations off the oracle's SwiGLU, first {bad[:3]}"


def reference(c, tol, ids=None):
    ids = c["ids"] if ids is None else ids
    return oracle.moe_block(c["fmt"], *c["gu"], *c["dn"], ids, c["w"], c["x"], c["experts"], c["hidden"], c["dff"],
                            rounding_tol=tol)


def gate_up_reference(c, ids=None):
    ids = c["ids"] if ids is None else ids
    return oracle.moe_gemv(c["fmt"], *c["gu"], ids, c["x"], 0, c["experts"], 2 * c["dff"], c["hidden"])


def check_block(c, what, exact, ids=None):
    say(what)
    y, h, a = run_block(c, ids, act=True)
    check_activations(h, a, what)
    h_ref, h_abs = gate_up_reference(c, ids)
    if exact:
        h32 = h_ref.astype(np.float32)
        same = (h == h32) | (np.isnan(h) & np.isnan(h32))
        assert same.all(), f"{what}: {int((~same).sum())} gate/up values differ, first {np.argwhere(~same)[0]}"
    else:
        assert_within(h, h_ref, h_abs, f"{what} gate/up")
    y_ref, a_ref, amb = reference(c, ROUNDING_TOL_EXACT if exact else ROUNDING_TOL_CONTRACT, ids)
    with np.errstate(invalid="ignore"):
        ok = (np.isnan(y) & np.isnan(y_ref)) | (np.abs(y - y_ref) <= 1e-5 * a_ref + amb + 1e-6)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside; first {i}: gpu={y[i]!r} "
                             f"ref={y_ref[i]!r} abs={a_ref[i]!r} amb={amb[i]!r}")
    return y, y_ref


@pytest.mark.parametrize("tokens", [1, 4, 8])
def test_block_exact_mxfp4(tokens):
    """The 30B-A3B-like block (hidden 2048, expert width 768, 128 experts, top-8)."""
    check_block(synth.moe_block(tokens, seed=tokens, exact=True), f"block exact mxfp4 T={tokens}", True)


@pytest.mark.parametrize("fmt", [2, 3])
def test_block_exact_other_formats(fmt):
    check_block(synth.moe_block(3, seed=10 + fmt, fmt=fmt, experts=16, exact=True), f"block exact fmt={fmt}", True)


@pytest.mark.parametrize("tokens", [1, 5])
def test_block_normal_inputs(tokens):
    check_block(synth.moe_block(tokens, seed=20 + tokens), f"block normal mxfp4 T={tokens}", False)


@pytest.mark.parametrize("fmt", [2, 3])
def test_block_normal_inputs_other_formats(fmt):
    check_block(synth.moe_block(3, seed=26 + fmt, fmt=fmt, experts=16), f"block normal fmt={fmt}", False)


@pytest.mark.parametrize("fmt,experts,hidden,dff,topk,tokens", [
    (1, 16, 2080, 96, 6, 3),     # ragged hidden, 6 of 8 slots, narrow expert rows
    (1, 16, 512, 2048, 16, 2),   # 16 slots: activations fill the 64 KiB LDS budget
    (1, 4, 256, 64, 1, 8),       # one slot, eight tokens
    (2, 8, 1024, 160, 3, 5),     # MXFP8, 3 of 4 slots
    (3, 8, 768, 48, 2, 4),       # NVFP4 rows of 24 bytes
    (3, 16, 1040, 784, 5, 2),    # NVFP4, ragged both ways
])
def test_block_shapes(fmt, experts, hidden, dff, topk, tokens):
    c = synth.moe_block(tokens, seed=hidden + dff, fmt=fmt, experts=experts, hidden=hidden, dff=dff, topk=topk,
                        exact=True)
    check_block(c, f"block fmt={fmt} E={experts} H={hidden} dff={dff} topk={topk} T={tokens}", True)


def test_block_invalid_ids():
    c = synth.moe_block(3, seed=31, experts=16, hidden=512, dff=256, topk=4, exact=True)
    ids = c["ids"].copy()
    ids[1, 2] = -1
    ids[2, 0] = 16
    y, _ = check_block(c, "block invalid ids", True, ids)
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all() and np.isfinite(y[0]).all()


def test_block_repeated_ids():
    """One expert in several slots of a token (the down kernel reads it once per slot)."""
    c = synth.moe_block(2, seed=32, experts=8, hidden=512, dff=256, topk=4, exact=True)
    ids = np.array([[3, 3, 3, 3], [0, 5, 0, 5]], dtype=np.int32)
    check_block(c, "block repeated ids", True, ids)


def test_block_is_deterministic():
    c = synth.moe_block(4, seed=33)
    say("block determinism")
    y1, h1 = run_block(c)
    y2, h2 = run_block(c)
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all() and (h1.view(np.uint32) == h2.view(np.uint32)).all()


def test_route_then_block():
    """Router logits -> ids and weights on the GPU -> block, against the oracle's routing and block."""
    c = synth.moe_block(4, seed=34)
    logits = synth.router_logits(synth.streams(35)[2], 4, c["experts"])
    say("route -> block")
    ids, w = mxq.moe_route(dev_f32(logits), c["topk"], True)
    gc, gs, _ = c["gu"]
    dc, ds, _ = c["dn"]
    y = host(mxq.moe_block(1, dev_u8(gc), dev_u8(gs), dev_u8(dc), dev_u8(ds), ids, w, dev_bf16(c["x"])))
    ids_ref, w_ref = oracle.moe_route(logits, c["topk"], True)
    assert (host(ids) == ids_ref).all()
    c["w"] = w_ref.astype(np.float32)
    y_ref, a_ref, amb = reference(c, ROUNDING_TOL_CONTRACT, ids_ref)
    # the routing weights differ by at most 1e-5 relative: another 1e-5 abs_y
    assert (np.abs(y - y_ref) <= 2e-5 * a_ref + amb + 1e-6).all()


@pytest.mark.parametrize("fmt,experts,hidden,dff,topk,tokens,renorm", [
    (1, 128, 2048, 768, 8, 1, True),   # the 30B-A3B-like block
    (1, 128, 2048, 768, 8, 4, False),
    (1, 128, 2048, 768, 8, 8, True),
    (1, 40, 512, 256, 6, 3, True),     # fewer experts than lanes
    (2, 300, 512, 160, 3, 8, True),    # MXFP8, experts past 128 (sixteen logits per lane)
    (3, 1000, 256, 128, 16, 5, False), # NVFP4, 1000 experts, 16 slots
    (1, 6, 256, 64, 6, 2, True),       # every expert selected
])
def test_routed_block_matches_route_then_block(fmt, experts, hidden, dff, topk, tokens, renorm):
    """Routing in place in the gate/up kernel gives, bit for bit, the ids, weights, workspace and outputs of
    mxq_moe_route followed by mxq_moe_block; the ids and weights also against the oracle's routing."""
    c = synth.moe_block(tokens, seed=experts + topk, fmt=fmt, experts=experts, hidden=hidden, dff=dff, topk=topk)
    logits = route_case(experts * 7 + tokens, tokens, experts)
    gc, gs, gg = c["gu"]
    dc, ds, dg = c["dn"]
    say(f"routed block fmt={fmt} E={experts} H={hidden} dff={dff} topk={topk} T={tokens} renorm={renorm}")
    banks = (dev_u8(gc), dev_u8(gs), dev_u8(dc), dev_u8(ds))
    x = dev_bf16(c["x"])
    lg = dev_f32(logits)
    n_ws = mxq.moe_block_workspace_elems(tokens, topk, dff)
    ws1 = torch.full((n_ws,), float("nan"), dtype=torch.float32, device="cuda:0")
    ws2 = torch.full((n_ws,), float("nan"), dtype=torch.float32, device="cuda:0")
    ids1, w1 = mxq.moe_route(lg, topk, renorm)
    y1 = mxq.moe_block(fmt, *banks, ids1, w1, x, gu_global_scale=dev_f32(gg), dn_global_scale=dev_f32(dg), h=ws1)
    y2, ids2, w2 = mxq.moe_block_routed(fmt, *banks, lg, topk, x, renorm=renorm, gu_global_scale=dev_f32(gg),
                                        dn_global_scale=dev_f32(dg), h=ws2)
    ids1, w1, ids2, w2 = host(ids1), host(w1), host(ids2), host(w2)
    assert (ids1 == ids2).all(), (ids1, ids2)
    assert (w1.view(np.uint32) == w2.view(np.uint32)).all(), (w1, w2)
    h1, a1 = (host(v.float()) if v.dtype == torch.bfloat16 else host(v)
              for v in mxq.moe_block_workspace_views(ws1, tokens, topk, dff))
    h2, a2 = (host(v.float()) if v.dtype == torch.bfloat16 else host(v)
              for v in mxq.moe_block_workspace_views(ws2, tokens, topk, dff))
    assert (h1.view(np.uint32) == h2.view(np.uint32)).all()
    assert (a1.view(np.uint32) == a2.view(np.uint32)).all()
    assert (host(y1).view(np.uint32) == host(y2).view(np.uint32)).all()
    ids_ref, w_ref = oracle.moe_route(logits, topk, renorm)
    assert (ids2 == ids_ref).all()
    assert (np.abs(w2 - w_ref) <= 1e-5 * w_ref + 1e-7).all()
