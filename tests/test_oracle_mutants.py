"""Plant plausible mistakes in copies of the C oracle (on the CPU) and check
that the pin suite rejects every one of them."""
import ctypes
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import oracle_pins as pins  # noqa: E402

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "quant_emax_fp4": ("const int emax = fmt == ORC_MXFP4 ? 2 : 8;", "const int emax = fmt == ORC_MXFP4 ? 3 : 8;"),
    "quant_emax_fp8": ("const int emax = fmt == ORC_MXFP4 ? 2 : 8;", "const int emax = fmt == ORC_MXFP4 ? 2 : 7;"),
    "quant_truncate": ("const double r = nearbyint(a / q) * q;", "const double r = floor(a / q) * q;"),
    "quant_ties_away": ("const double r = nearbyint(a / q) * q;", "const double r = round(a / q) * q;"),
    "quant_sign_dropped": ("| (neg << 3);", ";"),
    "quant_nv_scale_target": ("(float)amax / (6.0f * g);", "(float)amax / (4.0f * g);"),
    "nibble_order": ("(k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4)", "(k % 2 == 1) ? (byte & 0x0Fu) : (byte >> 4)"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * (double)m, (int)e - 1)", "ldexp(1.0 + 0.5 * (double)m, (int)e - 2)"),
    "e2m1_subnormal": ("0.5 * (double)m :", "1.0 * (double)m :"),
    "e2m1_sign": ("double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);\n    return s ? -mag : mag;",
                  "double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);\n    return mag;"),
    "e8m0_bias": ("ldexp(1.0, (int)u - 127)", "ldexp(1.0, (int)u - 126)"),
    "e4m3_bias": ("ldexp(1.0 + (double)m / 8.0, (int)e - 7)", "ldexp(1.0 + (double)m / 8.0, (int)e - 8)"),
    "e4m3_subnormal": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "mx_scale_index": ("orc_e8m0(scales_row[k / 32])", "orc_e8m0(scales_row[k / 16])"),
    "nv_scale_index": ("orc_e4m3(scales_row[k / 16])", "orc_e4m3(scales_row[k / 32])"),
    "nv_global_dropped": ("(q * s) * (double)g", "(q * s)"),
    "dropped_term": ("for (int64_t j = 0; j < k; ++j) {\n        double t", "for (int64_t j = 0; j < k - 1; ++j) {\n        double t"),
    "abs_sum": ("aacc += fabs(t);\n    }\n    *y = acc;", "aacc += t;\n    }\n    *y = acc;"),
    "gemm_abs_sum": ("aacc += fabs(t);\n                }", "aacc += t;\n                }"),
    "moe_x_index": ("x_per_slot ? x + p * k : x + t * k", "x_per_slot ? x + t * k : x + p * k"),
    "moe_expert_row": ("codes + (e * n + r) * cb", "codes + (r) * cb"),
    "gemm_row_index": ("X + rows[i] * k", "X + i * k"),
    "gemm_dropped_term": ("double t = (double)w[j] * orc_bf16(xr[j]);", "double t = (j + 1 < k) ? (double)w[j] * orc_bf16(xr[j]) : 0.0;"),
    "gemv_output_transposed": ("x + b * k, k, &y[b * n + r], &abs_y[b * n + r]", "x + b * k, k, &y[r * batch + b], &abs_y[r * batch + b]"),
    "bf16_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "route_tie_order": ("if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    "route_no_renorm": ("w[t * topk + s] /= sel;", "w[t * topk + s] /= 1.0;"),
    "route_softmax_shift": ("den += exp((double)l[e] - mx);", "den += exp((double)l[e]);"),
    "silu_sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "bf16_round_spacing": ("int q = (e < emin ? emin : e) - 8;", "int q = (e < emin ? emin : e) - 9;"),
    "block_silu_on_up": ("(double)(float)orc_silu(g32);", "(double)(float)orc_silu(u32);"),
    "block_weight_dropped": ("acc += ws * part;", "acc += part;"),
    "amb_one_side": ("dev[s * dff + j] = lo > hi ? lo : hi;", "dev[s * dff + j] = lo;"),
    "amb_half_interval": ("p_rel * fabs(p);", "0.5 * p_rel * fabs(p);"),
    "amb_weight_dropped": ("bacc += fabs(ws) * bpart;", "bacc += bpart;"),
    "block_no_bf16": ("a[s * dff + j] = orc_round_bf16(p);", "a[s * dff + j] = p;"),
    "block_fp64_swiglu": ("const double p = (double)(float)(s32 * u32);", "const double p = orc_silu(g32) * u32;"),
    "requant_tile_col": ("tile_scales[(r / bn) * tcols + col / bk]", "tile_scales[(r / bn) * tcols + col / bn]"),
    "requant_tile_row": ("tile_scales[(r / bn) * tcols + col / bk]", "tile_scales[(r / bk) * tcols + col / bk]"),
    "requant_scale_dropped": ("v[j] = (float)(orc_e4m3(codes_in[r * k + col]) * s);",
                              "v[j] = (float)(orc_e4m3(codes_in[r * k + col]));"),
    "requant_fp64_value": ("float v[32];\n            double amax = 0.0;\n            for (int j = 0; j < 32; ++j) {\n"
                           "                const int64_t col = b * 32 + j;\n"
                           "                const double s = (double)tile_scales[(r / bn) * tcols + col / bk];\n"
                           "                v[j] = (float)(orc_e4m3(codes_in[r * k + col]) * s);",
                           "double v[32];\n            double amax = 0.0;\n            for (int j = 0; j < 32; ++j) {\n"
                           "                const int64_t col = b * 32 + j;\n"
                           "                const double s = (double)tile_scales[(r / bn) * tcols + col / bk];\n"
                           "                v[j] = (orc_e4m3(codes_in[r * k + col]) * s);"),
    "requant_emax": ("se = (e - 1) - 8;\n                if (se < -127) se = -127;\n                if (se > 127) se = 127;\n            }\n            scales[r * nb + b]",
                     "se = (e - 1) - 7;\n                if (se < -127) se = -127;\n                if (se > 127) se = 127;\n            }\n            scales[r * nb + b]"),
    "split_saturating_scale": ("while (amax > 448.0 * ldexp(1.0, e)) ++e;", "while (0) ++e;"),
    "split_no_second_term": ("const double m = orc_quant_mag(fabs(res[j]) / ldexp(1.0, eb), 3, -6, 448.0);",
                             "const double m = 0.0;"),
    "split_residual_sign": ("res[j] = v[j] - (neg ? -m : m) * ldexp(1.0, ea);", "res[j] = v[j] - m * ldexp(1.0, ea);"),
    "split_term2_scale": ("const int eb = orc_split_exponent(amax2);", "const int eb = orc_split_exponent(amax);"),
    "requant_sign": ("(uint8_t)(orc_e4m3_code(orc_quant_mag(fabs(p), 3, -6, 448.0)) | (neg << 7));",
                     "(uint8_t)(orc_e4m3_code(orc_quant_mag(fabs(p), 3, -6, 448.0)));"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib), str(path), "-lm"],
                   check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, monkeypatch, name):
    path = _build_mutant(tmp_path, name)
    real = oracle._load()
    mutant = ctypes.CDLL(path)
    for attr in ("orc_e2m1", "orc_e8m0", "orc_e4m3", "orc_bf16", "orc_num_threads", "orc_set_num_threads",
                 "orc_dequant", "orc_gemv", "orc_moe_gemv", "orc_gemm_rows", "orc_moe_route", "orc_silu",
                 "orc_round_bf16", "orc_moe_block", "orc_quantize", "orc_requant_fp8", "orc_split_e4m3"):
        fr, fm = getattr(real, attr), getattr(mutant, attr)
        fm.argtypes, fm.restype = fr.argtypes, fr.restype
    monkeypatch.setattr(oracle, "_lib", mutant)
    failed = []
    for cname, check in pins.all_checks():
        try:
            check()
        except AssertionError:
            failed.append(cname)
    assert failed, f"mutant {name} passed every pin"
