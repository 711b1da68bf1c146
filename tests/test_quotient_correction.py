"""The NVFP4 quantizer computes each element quotient RN(v / d) as
RN(q0 + RN(v - q0 d) y) with q0 = RN(v y) and y = RN(1/d), the second and
third steps by fma (Markstein's residual correction).  This test proves on the
CPU that the identity holds for every fp32 mantissa of d and every bf16
mantissa of v, which, scaled by powers of two that keep every intermediate a
normal number, is every operand pair that step receives; a copy without the
correction must fail, so the check itself can fail."""
import shutil
import subprocess
import tempfile
from pathlib import Path

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float bits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
int main(void) {
    long bad = 0;
#pragma omp parallel for reduction(+:bad) schedule(static)
    for (uint32_t m = 0; m < (1u << 23); ++m) {
        const float d = bits(0x3F800000u | m);
        const volatile float one = 1.0f;
        const float y = one / d;
        for (uint32_t vm = 0; vm < 128; ++vm) {
            const float v = bits(0x3F800000u | (vm << 16));
            const float q0 = v * y;
            const float r = fmaf(-q0, d, v);
            const float q = CORRECT;
            if (q != v / d) ++bad;
        }
    }
    printf("%ld\n", bad);
    return 0;
}
"""


def _mismatches(correct_expr):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    with tempfile.TemporaryDirectory() as d:
        src = Path(d) / "q.c"
        src.write_text(SRC.replace("CORRECT", correct_expr))
        exe = Path(d) / "q"
        subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe), str(src), "-lm"], check=True)
        out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=300)
        return int(out.stdout.strip())


def test_residual_step_gives_the_correctly_rounded_quotient():
    assert _mismatches("fmaf(r, y, q0)") == 0


def test_without_the_residual_step_quotients_differ():
    assert _mismatches("q0 + 0.0f * r") > 0
