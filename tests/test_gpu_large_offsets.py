"""64-bit offsets: weight tensors larger than 2^32 bytes (the talk's slide 10 lists
32-bit grid arithmetic among the bugs it fixed).  Inputs are drawn on the device from
seeded torch generators (4.3 GB of codes would take minutes through numpy and the
bus); the oracle recomputes rows sampled from the start, the middle and the last
rows, whose byte offsets lie past 2^31 and 2^32."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
import oracle
from gpu_util import assert_within, dev_bf16, dev_i32, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def device_weight(n, k, seed, lead=()):
    g = torch.Generator(device=DEV).manual_seed(seed)
    codes = torch.randint(0, 256, lead + (n, k // 2), dtype=torch.uint8, device=DEV, generator=g)
    scales = torch.randint(118, 131, lead + (n, k // 32), dtype=torch.uint8, device=DEV, generator=g)
    return codes, scales


def bf16_x(shape, seed):
    f = np.random.default_rng(seed).standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def sampled_rows(n):
    rng = np.random.default_rng(n)
    return np.unique(np.concatenate([[0, 1, n // 2, n - 2, n - 1], rng.choice(n, 40, replace=False),
                                     n - 1 - rng.choice(1000, 20, replace=False)]))


def test_dense_gemv_codes_past_4gib():
    n, k = 1 << 20, 8192  # 4,294,967,296 code bytes
    codes, scales = device_weight(n, k, 1)
    x = bf16_x((4, k), 2)
    rows = sampled_rows(n)
    ch, sh = host(codes[rows]), host(scales[rows])
    for batch in (1, 4):
        say("large gemv", n, k, batch)
        y = host(mxq.gemv(1, codes, scales, dev_bf16(x[:batch])))
        y_ref, a_ref = oracle.gemv(1, ch, sh, None, x[:batch], rows.size, k)
        assert_within(y[:, rows], y_ref, a_ref, f"gemv {n}x{k} B={batch}")
        assert np.isfinite(y).all()


def test_gemm_codes_past_4gib():
    n, k, m = 1 << 20, 8192, 48  # tile path (m > 32)
    codes, scales = device_weight(n, k, 3)
    x = bf16_x((m, k), 4)
    say("large gemm", m, n, k)
    Y = mxq.gemm(1, codes, scales, dev_bf16(x), out_dtype=torch.float32)
    cols = sampled_rows(n)
    ycols = host(Y[:, torch.from_numpy(cols).to(DEV)])
    Y_ref, A_ref = oracle.gemm_rows(1, host(codes[cols]), host(scales[cols]), None, x, np.arange(m), cols.size, k)
    assert_within(ycols, Y_ref, A_ref, "gemm rows past 4 GiB")


def test_moe_bank_offsets_past_4gib():
    E, n, k = 64, 8192, 16384  # 64 experts x 67 MB of codes: expert 63 starts past 2^32 bytes
    codes, scales = device_weight(n, k, 5, lead=(E,))
    ids = np.array([[63, 0, 40], [62, 63, 31]], dtype=np.int32)
    x = bf16_x((2, 3, k), 6)
    say("large moe bank", E, n, k)
    y = host(mxq.moe_gemv(1, codes, scales, dev_i32(ids), dev_bf16(x), 1))
    for t in range(2):
        for s in range(3):
            e = int(ids[t, s])
            y_ref, a_ref = oracle.gemv(1, host(codes[e]), host(scales[e]), None, x[t, s][None], n, k)
            assert_within(y[t, s][None], y_ref, a_ref, f"moe expert {e}")
