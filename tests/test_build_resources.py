"""The HIP kernels keep everything in registers: no kernel of the last build
spills vector registers or uses scratch memory (per-lane scratch turns the streaming
kernels' register-resident passes into memory traffic; an MXFP8 GEMM that spilled
ran at an eighth of the MXFP4 rate).  The figures are the compiler's own resource
remarks, recorded by the build."""
import json
import os

import pytest

from block_float_quantized_mxq_amd import _build


def _usage():
    if not os.path.exists(_build.RESOURCES):
        pytest.skip("no build record (run __graft_entry__.build() first)")
    with open(_build.RESOURCES) as f:
        return json.load(f)


def test_every_kernel_recorded():
    usage = _usage()
    assert len(usage) > 100, f"only {len(usage)} kernels recorded"
    for name in ("gemm_kernel", "moe_gemm_stream_kernel", "gemv_rows_kernel", "gemv_mfma_kernel", "moe_kernel",
                 "moe_down_kernel", "moe_route_kernel", "quantize_kernel", "requant_fp8_kernel", "dequant_kernel"):
        assert any(name in k for k in usage), f"{name} missing from the build record"


def test_no_spills_or_scratch():
    # (scalar-register spills go to lanes of vector registers, not to memory: not counted)
    bad = {k: v for k, v in _usage().items() if v.get("scratch", 0) or v.get("vgpr_spill", 0)}
    assert not bad, f"{len(bad)} kernels spill or use scratch: " + "; ".join(
        f"{v['source']} {k[:90]} {v}" for k, v in list(bad.items())[:5])
