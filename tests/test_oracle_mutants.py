"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/qref.c``, plants one mistake in the copy (a dropped
term, a wrong sign, index or nibble, a transposed operand, a wrong tie rule),
builds it, swaps it in for the real oracle and checks that at least one of
the named pins in ``test_oracle.py`` now fails.  Nothing here touches a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import oracle
import tests.test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "qref.c")

MUTANTS = [
    ("q4k nibble halves swapped", "q[64 * g + l] = b & 15;", "q[64 * g + l] = b >> 4;",
     ["test_q4k_field_roundtrip", "test_q4k_special_cases"]),
    ("q4k min term dropped", "xval r = {a - b, e0, 0, a < b};", "xval r = {a, e0, 0, 0};",
     ["test_q4k_special_cases"]),
    ("q4k min sign flipped", "xval r = {a - b, e0, 0, a < b};", "xval r = {a + b, e0, 0, 0};",
     ["test_q4k_special_cases"]),
    ("q4k high scale bits from the wrong byte", "((s12[j] >> 6) << 4));", "((s12[j + 4] >> 6) << 4));",
     ["test_q4k_field_roundtrip"]),
    ("q4k sub-block index off", "int j = k / 32;", "int j = k / 64;", ["test_q4k_special_cases"]),
    ("q4k extra binary32 rounding", "xval r = {a - b, e0, 0, a < b};", "xval r = rn_f32(a - b, e0);",
     ["test_q4k_single_rounding"]),
    ("q6k scale per 32 weights", "s[k / 16]", "s[k / 32]", ["test_q6k_special_cases"]),
    ("q6k offset 31", "{nd * s * (q - 32), ed, 0, 0}", "{nd * s * (q - 31), ed, 0, 0}", ["test_q6k_special_cases"]),
    ("q6k high pair shift", "(qh[32 * h + l] >> (2 * r)) & 3", "(qh[32 * h + l] >> r) & 3",
     ["test_q6k_field_roundtrip"]),
    ("w4a16 symmetric zero-point 7", "zeros[gi * N + n] : 8", "zeros[gi * N + n] : 7", ["test_w4a16_special_cases"]),
    ("w4a16 group index by N", "int64_t gi = k / group;", "int64_t gi = (k + 1) / group;",
     ["test_w4a16_special_cases"]),
    ("gemm reversed K walk", "acc += xr[k] * wr[k];", "acc += xr[k] * wr[K - 1 - k];",
     ["test_gemm_matches_numpy"]),
    ("gemm bound signed", "bnd += fabs(xr[k]) * fabs(wr[k]);", "bnd += xr[k] * fabs(wr[k]);",
     ["test_gemm_matches_numpy", "test_gemm_smallest_shapes_exact_rationals"]),
    ("gemm accumulates in binary32", "acc += xr[k] * wr[k];", "acc = (float)(acc + xr[k] * wr[k]);",
     ["test_gemm_smallest_shapes_exact_rationals"]),
    ("gemm drops the last k", "for (int64_t k = 0; k < K; k++) {\n                acc += xr[k] * wr[k];",
     "for (int64_t k = 0; k < K - 1; k++) {\n                acc += xr[k] * wr[k];",
     ["test_gemm_smallest_shapes_exact_rationals", "test_gemm_matches_numpy"]),
    ("ties away from zero", "if (rem > half || (rem == half && (q & 1))) q++;", "if (rem >= half) q++;",
     ["test_rn_f16_matches_numpy"]),
    ("fragment-major halves and rows transposed", "((k / 8) % 2 * 32 + m % 32) * 8", "((m % 32) * 2 + (k / 8) % 2) * 8",
     ["test_fragment_major_is_an_axis_permutation", "test_fragment_major_operand_blocks"]),
    ("fragment-major padding rows not cleared", "out[idx] = m < M ? X[m * K + k] : 0;",
     "if (m < M) out[idx] = X[m * K + k];", ["test_fragment_major_is_an_axis_permutation"]),
    ("i8 ties away from zero", "return fmod(f, 2.0) == 0.0 ? f : f + 1.0;", "return f + 1.0;",
     ["test_i8_codes_ties_and_range"]),
    ("i8 scale over 255 levels", "*r = (float)(127.0 / amax);", "*r = (float)(255.0 / amax);",
     ["test_i8_scales_exact_rationals", "test_i8_codes_ties_and_range"]),
    ("i8 output scale inverted", "*s = (float)(amax / 127.0);", "*s = (float)(127.0 / amax);",
     ["test_i8_scales_exact_rationals", "test_gemm_i8_chain_close_to_fp64_product"]),
    ("i8 scale floor moved", "if (amax < ldexp(1.0, -96)) {", "if (amax < ldexp(1.0, -95)) {",
     ["test_i8_codes_ties_and_range"]),
    ("i8 gemm drops the weight scale", "xval sc = rn_f32(x.n * w.n, x.e + w.e);", "xval sc = x;",
     ["test_gemm_i8_scaled_matches_numpy_binary32"]),
    ("i8 gemm weight codes transposed", "acc += (int64_t)Qx[m * K + k] * Qw[k * N + n];",
     "acc += (int64_t)Qx[m * K + k] * Qw[n * K + k];", ["test_gemm_i8_unit_scales_is_integer_dot"]),
    ("i8 binary32 weights rounded to bf16", "xval r = rn_f32(v.n, v.e);", "xval r = rn_bf16(v.n, v.e);",
     ["test_dequant_f32_matches_exact"]),
    ("i8 fragment-major halves and rows transposed", "(k / 16) % 2 * 512 + m % 32 * 16",
     "m % 32 * 32 + (k / 16) % 2 * 16", ["test_fragment_major_i8_is_an_axis_permutation"]),
    ("fp16 subnormal grid wrong", "static xval rn_f16(int64_t n, int e) { return round_exact(n, e, 11, -14, 15); }",
     "static xval rn_f16(int64_t n, int e) { return round_exact(n, e, 11, -15, 15); }",
     ["test_rn_f16_matches_numpy"]),
]


@pytest.mark.parametrize("name,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, monkeypatch, name, old, new, catchers):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutant = tmp_path / "qref_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libqref_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(lib),
                           str(mutant), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(str(lib)))
    caught = []
    for fn_name in catchers:
        fn = getattr(pins, fn_name)
        params = [oracle.F16, oracle.BF16] if "dtype" in fn.__code__.co_varnames[:fn.__code__.co_argcount] else [None]
        for p in params:
            try:
                if p is None:
                    if "shape" in fn.__code__.co_varnames[:fn.__code__.co_argcount]:
                        fn(oracle.F16, (5, 48, 512))
                    elif fn.__code__.co_varnames[:fn.__code__.co_argcount] == ("M", "K"):
                        fn(40, 384)
                    elif fn.__code__.co_varnames[:fn.__code__.co_argcount] == ("fmt",):
                        fn("q4k")
                    else:
                        fn()
                else:
                    if "shape" in fn.__code__.co_varnames[:fn.__code__.co_argcount]:
                        fn(p, (5, 48, 512))
                    elif fn.__code__.co_varnames[:fn.__code__.co_argcount] == ("fmt", "sym", "dtype"):
                        fn("q4k", False, p)
                    else:
                        fn(p)
            except (AssertionError, ValueError):
                caught.append(fn_name)
                break
    assert caught, f"planted mistake '{name}' passed every pin in {catchers}"
