"""The C ABI without a GPU: the library loads, exports every function that
include/mxq.h declares, and rejects bad arguments on the host (validation runs
before any HIP call, so bogus-but-aligned pointer values are never touched)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")

import block_float_quantized_mxq_amd as mxq  # noqa: E402

OK, NULLPTR, SHAPE, ALIGN, FORMAT, UNSUPPORTED, DEVICE = 0, 1, 2, 3, 4, 5, 6
A = 0x10000  # aligned fake device address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mxq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["mxq_gemv", "mxq_gemv_config", "mxq_moe_gemv", "mxq_gemm", "mxq_dequant", "mxq_moe_route", "mxq_moe_block",
         "mxq_moe_block_noalloc", "mxq_moe_block_routed", "mxq_moe_gemm", "mxq_quantize", "mxq_requant_fp8", "mxq_stream_read",
         "mxq_status_string",
         "mxq_abi_version"])


def test_library_exports_every_declared_symbol():
    lib = mxq.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", mxq.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\b(mxq_\w+)\b", out.stdout))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.mxq_abi_version() == 9


def test_status_strings():
    for s in range(8):
        assert mxq.status_string(s)
    assert mxq.status_string(99) == "unknown status"


def gemv(fmt=1, codes=A, scales=A, g=None, x=A, y=A, n=8, k=64, batch=1):
    return mxq.lib().mxq_gemv(fmt, codes, scales, g, x, y, n, k, batch, None)


def moe(fmt=1, codes=A, scales=A, g=None, ids=A, x=A, per=0, y=A, E=4, n=8, k=64, T=1, topk=2):
    return mxq.lib().mxq_moe_gemv(fmt, codes, scales, g, ids, x, per, y, E, n, k, T, topk, None)


def gemm(fmt=1, codes=A, scales=A, g=None, x=A, y=A, ydt=0, m=4, n=8, k=64):
    return mxq.lib().mxq_gemm(fmt, codes, scales, g, x, y, ydt, m, n, k, None)


def deq(fmt=1, codes=A, scales=A, g=None, w=A, rows=4, k=64):
    return mxq.lib().mxq_dequant(fmt, codes, scales, g, w, rows, k, None)


def route(logits=A, ids=A, w=A, T=1, E=8, topk=2, renorm=0):
    return mxq.lib().mxq_moe_route(logits, ids, w, T, E, topk, renorm, None)


def block(fmt=1, codes=A, scales=A, g=None, dn_codes=A, dn_scales=A, dn_g=None, ids=A, w=A, x=A, h=A, y=A,
          E=4, hidden=64, dff=64, T=1, topk=2):
    return mxq.lib().mxq_moe_block(fmt, codes, scales, g, dn_codes, dn_scales, dn_g, ids, w, x, h, y,
                                   E, hidden, dff, T, topk, None)


def block_na(fmt=1, codes=A, scales=A, g=None, dn_codes=A, dn_scales=A, dn_g=None, ids=A, w=A, x=A, y=A,
             E=4, hidden=64, dff=64, T=1, topk=2):
    return mxq.lib().mxq_moe_block_noalloc(fmt, codes, scales, g, dn_codes, dn_scales, dn_g, ids, w, x, y,
                                           E, hidden, dff, T, topk, None)


def block_rt(fmt=1, codes=A, scales=A, g=None, dn_codes=A, dn_scales=A, dn_g=None, logits=A, renorm=0, ids=A, w=A,
             x=A, h=A, y=A, E=4, hidden=64, dff=64, T=1, topk=2):
    return mxq.lib().mxq_moe_block_routed(fmt, codes, scales, g, dn_codes, dn_scales, dn_g, logits, renorm, ids, w,
                                          x, h, y, E, hidden, dff, T, topk, None)


def mgemm(fmt=1, codes=A, scales=A, g=None, ids=A, x=A, per=0, y=A, ydt=0, ws=A, E=4, m=3, n=8, k=64, topk=2):
    return mxq.lib().mxq_moe_gemm(fmt, codes, scales, g, ids, x, per, y, ydt, ws, E, m, n, k, topk, None)


def quant(fmt=1, x=A, g=None, codes=A, scales=A, rows=4, k=64):
    return mxq.lib().mxq_quantize(fmt, x, g, codes, scales, rows, k, None)


@pytest.mark.parametrize("call", [gemv, moe, gemm, deq, block, block_na, block_rt, mgemm, quant])
def test_format_errors(call):
    assert call(fmt=0) == FORMAT
    assert call(fmt=4) == FORMAT
    assert call(fmt=3, g=None) == FORMAT      # NVFP4 needs its per-tensor scale
    assert call(fmt=1, g=A) == FORMAT         # MX formats take none
    assert call(fmt=2, g=A) == FORMAT


@pytest.mark.parametrize("call", [gemv, moe, gemm, deq, block, block_na, block_rt, mgemm])
def test_null_pointers(call):
    assert call(codes=None) == NULLPTR
    assert call(scales=None) == NULLPTR


def test_null_pointers_per_entry():
    assert gemv(x=None) == NULLPTR and gemv(y=None) == NULLPTR
    assert moe(ids=None) == NULLPTR and moe(x=None) == NULLPTR and moe(y=None) == NULLPTR
    assert gemm(x=None) == NULLPTR and gemm(y=None) == NULLPTR
    assert deq(w=None) == NULLPTR
    assert route(logits=None) == NULLPTR and route(ids=None) == NULLPTR and route(w=None) == NULLPTR
    for arg in ("dn_codes", "dn_scales", "ids", "w", "x", "h", "y"):
        assert block(**{arg: None}) == NULLPTR, arg
    for arg in ("dn_codes", "dn_scales", "ids", "w", "x", "y"):
        assert block_na(**{arg: None}) == NULLPTR, arg
    for arg in ("dn_codes", "dn_scales", "logits", "ids", "w", "x", "h", "y"):
        assert block_rt(**{arg: None}) == NULLPTR, arg
    for arg in ("ids", "x", "y", "ws"):
        assert mgemm(**{arg: None}) == NULLPTR, arg
    for arg in ("x", "codes", "scales"):
        assert quant(**{arg: None}) == NULLPTR, arg


def test_shape_errors():
    for bad in (0, -1):
        assert gemv(n=bad) == SHAPE and gemv(k=bad) == SHAPE and gemv(batch=bad) == SHAPE
        assert moe(E=bad) == SHAPE and moe(n=bad) == SHAPE and moe(T=bad) == SHAPE and moe(topk=bad) == SHAPE
        assert gemm(m=bad) == SHAPE and gemm(n=bad) == SHAPE and gemm(k=bad) == SHAPE
        assert deq(rows=bad) == SHAPE and deq(k=bad) == SHAPE
    # k must be a whole number of blocks: 32 for MX formats, 16 for NVFP4 (the GEMMs too)
    assert gemv(fmt=1, k=48) == SHAPE and gemv(fmt=2, k=16) == SHAPE
    assert gemv(fmt=3, g=A, k=40) == SHAPE
    assert moe(fmt=1, k=16) == SHAPE and deq(fmt=2, k=80) == SHAPE
    assert gemm(fmt=3, g=A, k=40) == SHAPE and gemm(fmt=1, k=48) == SHAPE and gemm(fmt=2, k=16) == SHAPE
    for bad in (0, -1):
        assert route(T=bad) == SHAPE and route(E=bad) == SHAPE and route(topk=bad) == SHAPE
        assert block(E=bad) == SHAPE and block(hidden=bad) == SHAPE and block(dff=bad) == SHAPE
        assert block(T=bad) == SHAPE and block(topk=bad) == SHAPE
        assert block_na(E=bad) == SHAPE and block_na(dff=bad) == SHAPE and block_na(T=bad) == SHAPE
    for bad in (0, -1):
        for arg in ("E", "hidden", "dff", "T", "topk"):
            assert block_rt(**{arg: bad}) == SHAPE, arg
    assert route(E=4, topk=5) == SHAPE                      # more picks than experts
    assert block_rt(E=4, topk=5) == SHAPE and block_rt(dff=80) == SHAPE
    assert block(hidden=48) == SHAPE and block(dff=80) == SHAPE
    assert block(fmt=3, g=A, dn_g=A, dff=40) == SHAPE
    # the two banks of one block share the format: its per-tensor scales go with it
    assert block(fmt=3, g=A, dn_g=None) == FORMAT and block(fmt=1, dn_g=A) == FORMAT
    for bad in (0, -1):
        for arg in ("E", "m", "n", "k", "topk"):
            assert mgemm(**{arg: bad}) == SHAPE, arg
    assert mgemm(k=48) == SHAPE and mgemm(fmt=3, g=A, k=24) == SHAPE  # whole blocks
    assert mgemm(ydt=2) == FORMAT
    for bad in (0, -1):
        assert quant(rows=bad) == SHAPE and quant(k=bad) == SHAPE
    assert quant(k=48) == SHAPE and quant(fmt=2, k=16) == SHAPE and quant(fmt=3, g=A, k=40) == SHAPE


def test_alignment_errors():
    assert gemv(codes=A + 8) == ALIGN and gemv(x=A + 2) == ALIGN and gemv(y=A + 2) == ALIGN
    assert gemv(fmt=3, g=A + 1, k=64) == ALIGN
    assert moe(ids=A + 2) == ALIGN and moe(codes=A + 4) == ALIGN and moe(x=A + 8) == ALIGN
    assert gemm(x=A + 4) == ALIGN and gemm(y=A + 1) == ALIGN
    assert deq(w=A + 2) == ALIGN and deq(codes=A + 1) == ALIGN
    assert route(logits=A + 2) == ALIGN and route(ids=A + 1) == ALIGN and route(w=A + 3) == ALIGN
    for arg, off in (("codes", 8), ("dn_codes", 4), ("x", 8), ("h", 4), ("y", 2), ("ids", 2), ("w", 1)):
        assert block(**{arg: A + off}) == ALIGN, arg
    assert block(fmt=3, g=A, dn_g=A + 2) == ALIGN
    for arg, off in (("codes", 8), ("dn_codes", 4), ("x", 8), ("y", 2), ("ids", 2), ("w", 1)):
        assert block_na(**{arg: A + off}) == ALIGN, arg
    for arg, off in (("codes", 8), ("dn_codes", 4), ("x", 8), ("h", 4), ("y", 2), ("ids", 2), ("w", 1),
                     ("logits", 2)):
        assert block_rt(**{arg: A + off}) == ALIGN, arg
    for arg, off in (("codes", 8), ("x", 8), ("y", 2), ("ids", 2), ("ws", 1)):
        assert mgemm(**{arg: A + off}) == ALIGN, arg
    assert quant(x=A + 8) == ALIGN and quant(codes=A + 8) == ALIGN and quant(fmt=3, g=A + 2, k=64) == ALIGN


def test_unsupported_sizes():
    assert gemv(batch=9) == UNSUPPORTED
    assert gemv(n=1 << 31) == UNSUPPORTED
    assert moe(T=9) == UNSUPPORTED and moe(topk=17) == UNSUPPORTED
    assert gemm(m=1 << 31) == UNSUPPORTED
    assert route(T=9) == UNSUPPORTED and route(E=1025, topk=2) == UNSUPPORTED and route(E=32, topk=17) == UNSUPPORTED
    assert block(T=9) == UNSUPPORTED and block(E=32, topk=17) == UNSUPPORTED
    # activations of the padded slot count staged in 64 KiB of LDS: 8 slots x 4096 x 2 bytes fit, 4128 do not
    assert block(topk=8, dff=4128) == UNSUPPORTED and block(topk=5, dff=4128) == UNSUPPORTED
    assert block(topk=4, dff=8224) == UNSUPPORTED and block(topk=2, dff=16416) == UNSUPPORTED
    assert block_na(T=9) == UNSUPPORTED and block_na(topk=8, dff=4128) == UNSUPPORTED
    assert block_rt(T=9) == UNSUPPORTED and block_rt(E=1025) == UNSUPPORTED and block_rt(topk=8, dff=4128) == UNSUPPORTED
    assert mgemm(topk=17) == UNSUPPORTED and mgemm(E=1025) == UNSUPPORTED
    assert mgemm(m=(1 << 24) // 8 + 1, topk=8) == UNSUPPORTED and mgemm(n=1 << 31) == UNSUPPORTED
    # every row streams, at any k (no staging of whole input rows)
    assert mgemm(fmt=3, g=A, k=4112) == DEVICE and mgemm(fmt=3, g=A, k=4080) == DEVICE
    assert mgemm(k=4096) == DEVICE and mgemm(fmt=3, g=A, k=8208) == DEVICE and mgemm(fmt=2, k=65536) == DEVICE
    assert quant(rows=1 << 20, k=(1 << 16) + 32) == UNSUPPORTED and quant(rows=1 << 31) == UNSUPPORTED


def gemv_cfg(config, **kw):
    import ctypes
    args = dict(fmt=1, codes=A, scales=A, g=None, x=A, y=A, n=8, k=64, batch=1)
    args.update(kw)
    c = ctypes.byref(mxq.GemvConfig(**config)) if config is not None else None
    return mxq.lib().mxq_gemv_config(args["fmt"], args["codes"], args["scales"], args["g"], args["x"], args["y"],
                                     args["n"], args["k"], args["batch"], c, None)


def test_gemv_config_argument_errors():
    assert gemv_cfg(None) == NULLPTR
    assert gemv_cfg(dict(), fmt=0) == FORMAT and gemv_cfg(dict(), n=0) == SHAPE
    assert gemv_cfg(dict(path=3)) == UNSUPPORTED and gemv_cfg(dict(path=-1)) == UNSUPPORTED
    assert gemv_cfg(dict(path=4), batch=5) == UNSUPPORTED and gemv_cfg(dict(rows_g=-1)) == UNSUPPORTED


def test_stream_read_argument_errors():
    sr = mxq.lib().mxq_stream_read
    assert sr(None, 16, 0, A, 4096, None) == NULLPTR and sr(A, 16, 0, None, 4096, None) == NULLPTR
    assert sr(A, 0, 0, A, 4096, None) == SHAPE and sr(A, 24, 0, A, 4096, None) == SHAPE
    assert sr(A, 16, 0, A, 0, None) == SHAPE and sr(A, 16, 2, A, 4096, None) == FORMAT
    assert sr(A + 8, 16, 1, A, 4096, None) == ALIGN and sr(A, 16, 1, A + 2, 4096, None) == ALIGN


def requant(ci=A, ts=A, co=A, sc=A, n=4, k=256, bn=128, bk=128):
    return mxq.lib().mxq_requant_fp8(ci, ts, co, sc, n, k, bn, bk, None)


def test_requant_argument_errors():
    for arg in ("ci", "ts", "co", "sc"):
        assert requant(**{arg: None}) == NULLPTR, arg
    for arg in ("n", "k", "bn", "bk"):
        assert requant(**{arg: 0}) == SHAPE and requant(**{arg: -1}) == SHAPE, arg
    assert requant(k=48) == SHAPE and requant(bk=48) == SHAPE  # whole 32-element blocks in one tile
    assert requant(ci=A + 8) == ALIGN and requant(co=A + 4) == ALIGN and requant(ts=A + 2) == ALIGN
    assert requant(n=1 << 20, k=(1 << 16) + 32) == UNSUPPORTED and requant(n=1 << 31) == UNSUPPORTED


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful where no GPU is present (it would launch on fake pointers)")
def test_device_error_without_gpu():
    assert gemv() == DEVICE and moe() == DEVICE and gemm() == DEVICE and deq() == DEVICE
    assert route() == DEVICE and block() == DEVICE and mgemm() == DEVICE
    assert mgemm(m=(1 << 24) // 8, topk=8, E=1024, k=4064) == DEVICE  # largest accepted sizes
    assert gemm(fmt=3, g=A, k=48) == DEVICE and mgemm(fmt=3, g=A, k=48) == DEVICE  # NVFP4 half-block rows
    assert quant() == DEVICE and quant(fmt=3, g=A, k=48) == DEVICE and quant(rows=1 << 20, k=1 << 16) == DEVICE
    assert block(topk=8, dff=4096) == DEVICE and block(topk=2, dff=16384) == DEVICE  # LDS budget exactly met
    # the largest workspace every admitted call needs (8 tokens x 16 slots x 2048 columns x 10 bytes) fits the array
    assert block_na() == DEVICE and block_na(T=8, topk=16, dff=2048, E=16) == DEVICE
    assert block_rt() == DEVICE and block_rt(E=1024, T=8, topk=16, dff=2048) == DEVICE
    assert gemv(fmt=3, g=A, k=48) == DEVICE  # NVFP4 rows of 24 bytes are valid too
    assert requant() == DEVICE and requant(n=1 << 20, k=1 << 16, bn=1, bk=32) == DEVICE
    assert gemv_cfg(dict()) == DEVICE and gemv_cfg(dict(path=4, mm_r=4, mm_s=2), batch=4) == DEVICE


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        mxq.gemv(1, torch.zeros(4, 16, dtype=torch.uint8), torch.zeros(4, 1, dtype=torch.uint8),
                 torch.zeros(1, 32, dtype=torch.bfloat16))
