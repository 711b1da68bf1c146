"""Helpers for the GPU parity tests: host arrays -> device tensors, and the
element-wise comparison against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def say(*args):
    """Name the case before a GPU step, flushed, so a failure points at it."""
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> bfloat16 device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_within(y_gpu, y_ref, abs_ref, what, rel=1e-5, atol=1e-6):
    """|y - y_ref| <= rel * sum|w x| + atol element by element (NaN matches NaN)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    ok = oracle.within_tolerance(y_gpu, y_ref, abs_ref, rel, atol)
    if not ok.all():
        idx = np.argwhere(~ok)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {idx.shape[0]} of {ok.size} outputs outside tolerance; first at {i}: "
                             f"gpu={y_gpu[i]!r} ref={y_ref[i]!r} bound={rel * abs_ref[i] + atol!r}")


def same_bits_f32(a, b):
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
