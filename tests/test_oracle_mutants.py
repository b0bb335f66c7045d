"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/rmsq_oracle.c (on the CPU,
in a temporary directory), builds it, and runs the pin tests of
test_oracle_codecs.py and test_oracle_pipeline.py against that build. Every
planted mistake must make at least one pin fail; the unmodified copy must
pass them all.
"""
import functools
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_codecs as TC
from tests import test_oracle_gemm as TG
from tests import test_oracle_pipeline as TP

SRC = os.path.join(os.path.dirname(oracle.__file__), "rmsq_oracle.c")

# name -> (text in the oracle, planted replacement)
MUTANTS = {
    "eps outside the square root": (
        "double denom = ss / (double)N + (double)eps;\n    double inv = denom > 0.0 ? 1.0 / sqrt(denom) : 0.0;",
        "double denom = ss / (double)N;\n    double inv = denom > 0.0 ? 1.0 / sqrt(denom) + (double)eps : 0.0;"),
    "mean over N - 1": ("ss / (double)N + (double)eps", "ss / (double)(N - 1) + (double)eps"),
    "no square root": ("1.0 / sqrt(denom)", "1.0 / denom"),
    "gamma dropped": ("double y = hbuf[j] * oracle_bf16_to_double(gamma[j]) * inv;", "double y = hbuf[j] * inv;"),
    "gamma as 1 + gamma": ("double y = hbuf[j] * oracle_bf16_to_double(gamma[j]) * inv;",
                           "double y = hbuf[j] * (1.0 + oracle_bf16_to_double(gamma[j])) * inv;"),
    "norm reads the unrounded residual sum": ("hbuf[j] = oracle_bf16_to_double(hb);", "hbuf[j] = sum;"),
    "y rounded to bf16 before gamma": (
        "double y = hbuf[j] * oracle_bf16_to_double(gamma[j]) * inv;",
        "double y = oracle_bf16_to_double(oracle_bf16_from_double(hbuf[j] * inv)) * oracle_bf16_to_double(gamma[j]);"),
    "fp8 maximum 240 (fnuz)": ("(float)(amax / 448.0)", "(float)(amax / 240.0)"),
    "e4m3 exponent bias 8": ("minifloat_code(a, -6, 3)", "minifloat_code(a, -7, 3)"),
    "ties away from zero": ("double k = nearbyint(ldexp(a, mbits - E));", "double k = round(ldexp(a, mbits - E));"),
    "subnormals flushed": ("    if (E < emin)\n        E = emin;", "    if (E < emin)\n        return 0;"),
    "bf16 rounds toward zero": ("uint32_t c = minifloat_code(a, -126, 7);",
                                "uint32_t c = minifloat_code(a * (1.0 - 0x1p-9), -126, 7);"),
    "e4m3fn not saturating": ("    if (c > 0x7E)\n        c = 0x7E;", "    if (c > 0x7F)\n        c = 0x7F;"),
    "negative zero loses its sign": ("uint8_t sign = signbit(v) ? 0x80 : 0;", "uint8_t sign = v < 0 ? 0x80 : 0;"),
    "zero group scale 0": ("amax == 0.0 ? 1.0f :", "amax == 0.0 ? 0.0f :"),
    "e2m1 saturating at 4": ("    if (c > 0x7)\n        c = 0x7;", "    if (c > 0x6)\n        c = 0x6;"),
    "e8m0 exponent off by one": ("int e = (e2 - 1) - 2;", "int e = (e2 - 1) - 1;"),
    "nibbles swapped": ("(uint8_t)(lo | (hi << 4))", "(uint8_t)(hi | (lo << 4))"),
    "tiled scale offset transposed": ("+ g * 32 + (m % 32);", "+ (m % 32) * groups_per_row + g;"),
    "column-major scales stored row-major": ("return g * M + m;", "return m * G + g;"),
    "GEMM weight nibbles swapped": ("uint8_t code = (uint8_t)((wr[k / 2] >> (4 * (k % 2))) & 0xF);",
                                    "uint8_t code = (uint8_t)((wr[k / 2] >> (4 * (1 - k % 2))) & 0xF);"),
    "GEMM e8m0 bias 126": ("return ldexp(1.0, (int)byte - 127);", "return ldexp(1.0, (int)byte - 126);"),
    "GEMM activation scale dropped": ("da[k] = oracle_e2m1_decode(code) * e8m0_value(ea[k / 32]);",
                                      "da[k] = oracle_e2m1_decode(code);"),
    "GEMM weight scale per 16": ("e8m0_value(sr[k / 32])", "e8m0_value(sr[(k / 16) % (K / 32)])"),
    "A16W8 activation scale dropped": ("da[k] = oracle_e4m3fn_decode(qa[k]) * (double)sa[k / 128];",
                                       "da[k] = oracle_e4m3fn_decode(qa[k]);"),
    "A16W8 weight block rows of 64": ("const float* sr = w_scale + (n / 128) * kb;",
                                      "const float* sr = w_scale + ((n / 64) % ((N + 127) / 128)) * kb;"),
    "A16W8 weight scale per 64 columns": ("(double)sr[k / 128]);", "(double)sr[(k / 64) % kb]);"),
    "AFP4 activation nibbles swapped": ("uint8_t c = (uint8_t)((arow[k / 2] >> (4 * (k % 2))) & 0xF);",
                                        "uint8_t c = (uint8_t)((arow[k / 2] >> (4 * (1 - k % 2))) & 0xF);"),
    "AFP4 activation scales always row-major": ("a_scale[scale_offset(m, k / 32, M, G, a_layout)]",
                                                "a_scale[scale_offset(m, k / 32, M, G, 0)]"),
    "A8W8 activation scale per 32 columns": ("scale_offset(m, k / 128, M, blocks, a_layout)",
                                             "scale_offset(m, (k / 32) % blocks, M, blocks, a_layout)"),
    "A8W8 weight block scale ignored": ("(oracle_e4m3fn_decode(wrow[k]) * (double)brow[k / 128]);",
                                        "(oracle_e4m3fn_decode(wrow[k]) * 1.0);"),
    "A16W8 weight scale divides": ("acc += da[k] * (oracle_e4m3fn_decode(wr[k]) * (double)sr[k / 128]);",
                                   "acc += da[k] * (oracle_e4m3fn_decode(wr[k]) / (double)sr[k / 128]);"),
}


def _pins():
    p = []
    for fn in (TC.test_bf16_overflow_and_signed_zero, TC.test_e4m3fn_hand_values, TC.test_e2m1_ties_and_saturation,
               TC.test_e2m1_decode_table, TC.test_e4m3fn_decode_matches_torch, TP.test_row_a_fp8_by_hand,
               TP.test_row_a_mxfp4_by_hand, TP.test_fp8_tie_heavy_group, TP.test_zero_row_and_zero_group,
               TP.test_tiny_workload_matches_exact_reference, TP.test_eps_is_inside_the_root_and_large_eps_matters,
               TP.test_fused_equals_the_unfused_chain, TP.test_tiled32_is_a_permutation_of_row_major,
               TP.test_column_major_scales_are_the_transpose, TP.test_row_stride_larger_than_n,
               TC.test_mx_scale_exponent_definition, TC.test_fp8_scale_is_ieee_fp32_division,
               TC.test_bf16_decode_every_pattern, TC.test_e4m3fn_encode_matches_torch_inside_range,
               TC.test_e2m1_encode_by_brute_force, TC.test_bf16_encode_matches_torch_on_fp32_patterns,
               TC.test_bf16_encode_doubles_by_nearest_search):
        p.append(fn)
    p += [functools.partial(TP.test_closed_form_rows, k=k) for k in (0, 2)]
    p += [functools.partial(TP.test_fp8_matches_exact_rational_reference, seed=0, residual=r) for r in (False, True)]
    p.append(functools.partial(TP.test_mxfp4_matches_exact_rational_reference, seed=0))
    p += [functools.partial(TC.test_e4m3fn_encode_every_bf16_by_brute_force, scale=s) for s in (1.0, 2.0 ** -7)]
    p += [TG.test_hand_example, TG.test_lossless_activations_match_numpy_matmul,
          TG.test_equals_its_own_quantization_times_the_weights]
    p += [functools.partial(TG.test_power_of_two_scaling, k=k) for k in (-7, 3)]
    p += [TG.test_a16w8_hand_example, TG.test_a16w8_lossless_activations_match_numpy_matmul,
          TG.test_a16w8_equals_its_own_quantization_times_the_weights]
    p += [TG.test_afp4wfp4_hand_example, TG.test_a8w8_hand_example]
    p += [functools.partial(TG.test_afp4wfp4_matches_numpy_dequant_matmul, layout=k) for k in (0, 1, 2)]
    p += [functools.partial(TG.test_a8w8_matches_numpy_dequant_matmul, layout=k) for k in (0, 2)]
    return p


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                    "-I", os.path.dirname(SRC), str(src), "-o", str(lib), "-lm"], check=True)
    return oracle.Oracle(str(lib))


def _first_failure(orc):
    for pin in _pins():
        try:
            pin(orc)
        except (AssertionError, ValueError):
            return getattr(pin, "func", pin).__name__
    return None


def test_unmodified_copy_passes_every_pin(tmp_path):
    assert _first_failure(_build(tmp_path, "clean", open(SRC).read())) is None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutant = _build(tmp_path, "mutant", text.replace(old, new))
    killer = _first_failure(mutant)
    assert killer is not None, f"no pin catches: {name}"
