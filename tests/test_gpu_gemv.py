"""Dense GEMV parity: HIP kernels (through the C ABI) against the CPU oracle,
element by element, |y - y_ref| <= 1e-5 * sum|w x| + 1e-6 on the fp32 output."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
import synth
from gpu_util import assert_within, dev_bf16, dev_f32, dev_u8, host, say

pytestmark = pytest.mark.gpu

FMT_NAMES = {1: "mxfp4", 2: "mxfp8", 3: "nvfp4"}


def run(case, x=None, config=None):
    x = case["x"] if x is None else x
    return host(mxq.gemv(case["fmt"], dev_u8(case["codes"]), dev_u8(case["scales"]), dev_bf16(x),
                         dev_f32(case["g"]), config=config))


def check_all(case, what, config=None):
    say(what)
    y = run(case, config=config)
    y_ref, a_ref = oracle.gemv(case["fmt"], case["codes"], case["scales"], case["g"], case["x"], case["n"], case["k"])
    assert_within(y, y_ref, a_ref, what)
    return y


def check_rows(case, rows, what, config=None):
    """Full-size launch; the oracle recomputes the sampled rows one by one."""
    say(what)
    y = run(case, config=config)
    y_ref, a_ref = oracle.gemv(case["fmt"], case["codes"][rows], case["scales"][rows], case["g"], case["x"],
                               rows.size, case["k"])
    assert_within(y[:, rows], y_ref, a_ref, what)
    assert np.isfinite(y).all()
    return y


def sample_rows(n, count=512, seed=0):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 15, 16, 63, 64, n // 2, n - 65, n - 64, n - 17, n - 16, n - 2, n - 1]
    rows = np.concatenate([rng.choice(n, size=min(count, n), replace=False), np.array(edges)])
    return np.unique(np.clip(rows, 0, n - 1))


def test_single_mxfp4_gemv_all_outputs():
    """512 x 1024 MXFP4, E8M0 U[120,130], one bf16 vector, seed 0."""
    check_all(synth.single_gemv(0), "single mxfp4 512x1024")


@pytest.mark.parametrize("which", ["gate_up", "down", "qkv"])
@pytest.mark.parametrize("batch", [1, 4])
def test_dense_layer_full_size_sampled(which, batch):
    case = synth.dense_layer(which, batch, seed=0)
    check_rows(case, sample_rows(case["n"]), f"dense {which} B={batch}")


@pytest.mark.parametrize("fmt", [2, 3])
def test_format_sweep_full_size_sampled(fmt):
    case = synth.format_sweep(fmt, seed=0)
    check_rows(case, sample_rows(case["n"]), f"format sweep {FMT_NAMES[fmt]} 5120x25600")


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("n,k", [(1000, 5120), (77, 25600), (300, 2048), (129, 768)])
def test_all_outputs_ragged(fmt, batch, n, k):
    """Several row tiles plus a ragged last tile, every output checked."""
    sc, ss, sx, _, _ = synth.streams(n + k + batch)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k)
    x = synth.bf16_normal(sx, (batch, k))
    check_all(dict(fmt=fmt, codes=codes, scales=scales, g=g, x=x, n=n, k=k),
              f"ragged {FMT_NAMES[fmt]} n={n} k={k} B={batch}")


@pytest.mark.parametrize("fmt,k", [(1, 32), (2, 32), (3, 16), (3, 48), (3, 32), (1, 96), (3, 4112)])
@pytest.mark.parametrize("n", [1, 7, 5119])
def test_small_k_and_row_tails_with_guard(fmt, k, n):
    """Tiny and odd K (NVFP4 rows of 8/24 bytes), odd N; nothing past y is written."""
    sc, ss, sx, _, _ = synth.streams(3 * n + k)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k)
    x = synth.bf16_normal(sx, (2, k))
    say("tails", fmt, n, k)
    guard = 4099
    big = torch.full((2 * n + guard,), 12345.0, dtype=torch.float32, device="cuda:0")
    out = big[: 2 * n].view(2, n)
    mxq.gemv(fmt, dev_u8(codes), dev_u8(scales), dev_bf16(x), dev_f32(g), out=out)
    b = host(big)
    assert (b[2 * n:] == 12345.0).all(), "kernel wrote past the end of y"
    y_ref, a_ref = oracle.gemv(fmt, codes, scales, g, x, n, k)
    assert_within(b[: 2 * n].reshape(2, n), y_ref, a_ref, f"tails fmt={fmt} n={n} k={k}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_one_hot_is_exact(fmt):
    """x = e_j: one nonzero term, so y[i] = w[i][j] exactly (nibble order, block and scale indexing)."""
    n, k = 64, 256
    sc, ss, _, _, _ = synth.streams(40 + fmt)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k)
    w = oracle.dequant(fmt, codes, scales, g, n, k)
    cols = list(range(0, 40)) + [63, 64, 127, 128, 200, 255]
    x = np.zeros((len(cols), k), dtype=np.uint16)
    for b in range(0, len(cols), 8):
        xb = np.zeros((min(8, len(cols) - b), k), dtype=np.uint16)
        for i, j in enumerate(cols[b:b + 8]):
            xb[i, j] = 0x3F80
        say("one-hot", fmt, cols[b:b + 8])
        y = host(mxq.gemv(fmt, dev_u8(codes), dev_u8(scales), dev_bf16(xb), dev_f32(g)))
        for i, j in enumerate(cols[b:b + 8]):
            assert (y[i] == w[:, j]).all(), (fmt, j)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_sign_flip_and_zero_codes(fmt):
    """Toggling every code's sign bit negates y (to the acceptance bound: the bf16 dot
    instruction does not round symmetrically, so bitwise negation is not guaranteed);
    all-zero codes give exactly zero."""
    n, k = 333, 2048
    sc, ss, sx, _, _ = synth.streams(50 + fmt)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k)
    x = synth.bf16_normal(sx, (3, k))
    flip = codes ^ (np.uint8(0x80) if fmt == 2 else np.uint8(0x88))
    say("sign flip", fmt)
    y = host(mxq.gemv(fmt, dev_u8(codes), dev_u8(scales), dev_bf16(x), dev_f32(g)))
    yf = host(mxq.gemv(fmt, dev_u8(flip), dev_u8(scales), dev_bf16(x), dev_f32(g)))
    _, a_ref = oracle.gemv(fmt, codes, scales, g, x, n, k)
    assert_within(-yf.astype(np.float64), y.astype(np.float64), 2 * a_ref, f"sign flip fmt={fmt}")
    zero = np.zeros_like(codes)
    y0 = host(mxq.gemv(fmt, dev_u8(zero), dev_u8(scales), dev_bf16(x), dev_f32(g)))
    assert (y0 == 0).all()


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_scale_bump_doubles_block_contribution(fmt):
    """Block b's scale exponent +1: y' - y equals that block's contribution (within tolerance)."""
    n, k = 256, 1024
    sc, ss, sx, _, _ = synth.streams(60 + fmt)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k)
    x = synth.bf16_normal(sx, (1, k))
    b = 5
    bumped = scales.copy()
    if fmt == 3:
        bumped[:, b] = (scales[:, b] & 0x87) | (7 << 3)
        scales = bumped.copy()
        bumped[:, b] = scales[:, b] + 8
    else:
        bumped[:, b] = scales[:, b] + 1
    bs = 16 if fmt == 3 else 32
    cpb = bs if fmt == 2 else bs // 2
    iso = np.zeros_like(codes)
    iso[:, b * cpb:(b + 1) * cpb] = codes[:, b * cpb:(b + 1) * cpb]
    say("scale bump", fmt)
    yi0 = host(mxq.gemv(fmt, dev_u8(iso), dev_u8(scales), dev_bf16(x), dev_f32(g)))
    yi1 = host(mxq.gemv(fmt, dev_u8(iso), dev_u8(bumped), dev_bf16(x), dev_f32(g)))
    assert (yi1 == 2 * yi0).all()  # powers of two commute with rounding
    y0 = host(mxq.gemv(fmt, dev_u8(codes), dev_u8(scales), dev_bf16(x), dev_f32(g)))
    y1 = host(mxq.gemv(fmt, dev_u8(codes), dev_u8(bumped), dev_bf16(x), dev_f32(g)))
    _, a_ref = oracle.gemv(fmt, codes, bumped, g, x, n, k)
    assert_within(y1.astype(np.float64) - y0, yi0.astype(np.float64), 2 * a_ref, "scale bump")


def test_format_dispatch_is_per_format():
    """MXFP8 bytes read through the MXFP4 path must not reproduce the MXFP8 result."""
    n, k = 64, 512
    sc, ss, sx, _, _ = synth.streams(70)
    codes, scales, _ = synth.weights(2, sc, ss, n, k)
    x = synth.bf16_normal(sx, (1, k))
    say("dispatch")
    y8 = host(mxq.gemv(2, dev_u8(codes), dev_u8(scales), dev_bf16(x)))
    as4 = codes.reshape(n, k)[:, : k // 2]  # same bytes, half the row, as E2M1 pairs
    y4 = host(mxq.gemv(1, dev_u8(np.ascontiguousarray(as4)), dev_u8(scales), dev_bf16(x)))
    y_ref, a_ref = oracle.gemv(2, codes, scales, None, x, n, k)
    assert_within(y8, y_ref, a_ref, "mxfp8")
    assert not oracle.within_tolerance(y4, y_ref, a_ref).all()


def test_deterministic_bit_identical():
    case = synth.dense_layer("down", 4, seed=1)
    say("determinism")
    codes, scales, x = dev_u8(case["codes"]), dev_u8(case["scales"]), dev_bf16(case["x"])
    y1 = host(mxq.gemv(1, codes, scales, x))
    for _ in range(3):
        assert (host(mxq.gemv(1, codes, scales, x)).view(np.uint32) == y1.view(np.uint32)).all()


def test_rejects_bad_arguments_on_gpu():
    codes = torch.zeros(8, 16, dtype=torch.uint8, device="cuda:0")
    scales = torch.zeros(8, 1, dtype=torch.uint8, device="cuda:0")
    x = torch.zeros(9, 32, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(mxq.MxqError) as e:
        mxq.gemv(1, codes, scales, x)  # batch 9 > 8: rejected by the C library
    assert e.value.status == 5
    with pytest.raises(ValueError):
        mxq.gemv(3, codes, torch.zeros(8, 2, dtype=torch.uint8, device="cuda:0"), x[:1])  # NVFP4 without g


# Matrix-unit GEMV settings (row blocks per wave, k split, waves per workgroup).
MFMA_SETTINGS = [(1, 1, 4), (2, 1, 4), (4, 1, 4), (1, 2, 4), (1, 4, 4), (2, 4, 4), (4, 4, 4), (2, 8, 8)]


@pytest.mark.parametrize("setting", MFMA_SETTINGS)
@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("n,k", [(1000, 5120), (77, 25600), (129, 768), (300, 96), (64, 4096)])
def test_matrix_unit_settings_all_outputs(setting, fmt, n, k):
    """Every compiled (rows per wave, k split, waves) setting of the matrix-unit
    GEMV, forced for batches 1, 3 and 8, every output checked (ragged row
    blocks, k ranges that end inside a pass, empty k ranges)."""
    r, ks, nw = setting
    config = dict(path=1, mfma_r=r, mfma_ks=ks, mfma_nw=nw)
    sc, ss, sx, _, _ = synth.streams(7 * n + k + fmt)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k)
    for batch in (1, 3, 8):
        x = synth.bf16_normal(sx, (batch, k))
        check_all(dict(fmt=fmt, codes=codes, scales=scales, g=g, x=x, n=n, k=k),
                  f"matrix unit {setting} {FMT_NAMES[fmt]} n={n} k={k} B={batch}", config)


# Matrix-mode rows (four-row groups per lane, k split across waves).
MM_SETTINGS = [(4, 1), (4, 2), (4, 4), (2, 2), (2, 4)]


@pytest.mark.parametrize("setting", MM_SETTINGS)
@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("n,k", [(1000, 5120), (77, 25600), (129, 768), (300, 96), (5, 4112)])
def test_matrix_mode_settings_all_outputs(setting, fmt, n, k):
    """Every compiled matrix-mode setting (16 x 16 x 32 MFMA on the FMA-mode
    loads), forced for batches 1 .. 4, every output checked: ragged row groups,
    rows shorter than one pass, NVFP4 rows of 8-byte chunks (k = 4112)."""
    config = dict(path=4, mm_r=setting[0], mm_s=setting[1])
    if k % (16 if fmt == 3 else 32):
        k += 16  # MX formats: whole 32-element blocks
    sc, ss, sx, _, _ = synth.streams(11 * n + k + fmt)
    codes, scales, g = synth.weights(fmt, sc, ss, n, k)
    for batch in (1, 2, 3, 4):
        x = synth.bf16_normal(sx, (batch, k))
        check_all(dict(fmt=fmt, codes=codes, scales=scales, g=g, x=x, n=n, k=k),
                  f"matrix mode {setting} {FMT_NAMES[fmt]} n={n} k={k} B={batch}", config)


def test_every_path_at_full_size():
    """Each GEMV path (matrix unit, FMA rows, matrix-mode rows) forced on the same
    full-size gate/up input at batches 1 and 4: each within the acceptance bound
    of the oracle on sampled rows."""
    for batch in (1, 4):
        case = synth.dense_layer("gate_up", batch, seed=3)
        rows = sample_rows(case["n"], 256, seed=3)
        for path in (1, 2, 4):
            check_rows(case, rows, f"gate/up B={batch} path {path}", dict(path=path))


def test_config_entry_point_rejects_uncompiled_settings():
    case = synth.single_gemv(0)
    with pytest.raises(mxq.MxqError) as e:
        run(case, config=dict(path=2, rows_g=16, rows_s=3, rows_r=2))  # k split 3 is not compiled
    assert e.value.status == 5
    with pytest.raises(mxq.MxqError) as e:
        run(case, config=dict(path=7))
    assert e.value.status == 5
