"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/gemm_oracle.c`` to a temporary directory, plants one
mistake by a textual edit (a dropped term, a wrong sign, a transposed index,
a detour through fp32, flushed subnormals, ties rounded away, a wrong zero
sign, saturation instead of infinity; in the fused epilogue a bias per row,
beta or alpha on the wrong term, a transposed C, a rounding before the
epilogue; in FP8 a wrong exponent bias, flushed subnormals, the other NaN
convention, saturation in place of infinity, swapped formats, a rounding
before the scale; with per-channel scales a scale per row, a dropped
activation scale, a rounding before the scale; with an fp16 running sum a
chunk of 32, chunks counted from k = 0, one rounding per update instead of
the chunk's and the addition's, a wide running sum, a dropped chunk, a wrong sign, a wrong row of B), compiles the copy with gcc, points the oracle wrapper at it
and runs the pin battery.  At least one pin must fail for every planted mistake.  All
of this runs on the CPU; the real oracle is not modified.
"""
from __future__ import annotations

import ctypes
import shutil
import subprocess
from pathlib import Path

import pytest

import oracle
from tests import test_oracle_acc16_pins as hpins
from tests import test_oracle_bf16_pins as bpins
from tests import test_oracle_epilogue_pins as epins
from tests import test_oracle_fp8_pins as fpins
from tests import test_oracle_pins as pins

SRC = Path(oracle.__file__).resolve().parent / "gemm_oracle.c"

MUTATIONS = {
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k)\n        acc += g_lut[arow[k]]",
                          "for (int64_t k = 0; k + 1 < K; ++k)\n        acc += g_lut[arow[k]]"),
    "wrong_sign": ("acc += g_lut[arow[k]] * g_lut[brow[k]];", "acc -= g_lut[arow[k]] * g_lut[brow[k]];"),
    "transposed_output": ("D[m * N + n] = entry(", "D[n * M + m] = entry("),
    "b_row_index": ("D[m * N + n] = entry(A + m * K, B + n * K, K);",
                    "D[m * N + n] = entry(A + m * K, B + ((n + 1) % N) * K, K);"),
    "round_via_fp32": ("return f16_encode_rne(dot(arow, brow, K));",
                       "return f16_encode_rne((double)(float)dot(arow, brow, K));"),
    "flush_subnormals": ("v = ldexp((double)frac, -24);", "v = 0.0 * frac;"),
    "ties_away": ("    if (rem > 0.5 || (rem == 0.5 && (n & 1)))\n        n += 1;\n    if (n == 2048)",
                  "    if (rem >= 0.5)\n        n += 1;\n    if (n == 2048)"),
    "negative_zero_start": ("double acc = 0.0;\n    for (int64_t k = 0; k < K; ++k)\n        acc += g_lut[arow[k]]",
                            "double acc = -0.0;\n    for (int64_t k = 0; k < K; ++k)\n        acc += g_lut[arow[k]]"),
    "saturating_overflow": ("if (E > 15)\n        return sign | 0x7c00;\n    if (n < 1024)",
                            "if (E > 15)\n        return sign | 0x7bff;\n    if (n < 1024)"),
    # fused epilogue
    "bias_per_row": ("r = r + g_lut[bias[n]];", "r = r + g_lut[bias[m % N]];"),
    "beta_scales_bias": ("r = r + g_lut[bias[n]];", "r = r + b * g_lut[bias[n]];"),
    "alpha_scales_c": ("r = r + b * g_lut[C[m * N + n]];", "r = r + a * b * g_lut[C[m * N + n]];"),
    "c_transposed": ("r = r + b * g_lut[C[m * N + n]];", "r = r + b * g_lut[C[(n * M + m) % (M * N)]];"),
    "epilogue_double_rounding": ("double r = a * dot(A + m * K, B + n * K, K);",
                                 "double r = a * g_lut[f16_encode_rne(dot(A + m * K, B + n * K, K))];"),
    # bfloat16
    "bf16_exponent_bias": ("v = ldexp((double)(128 + frac), expo - 134);",
                           "v = ldexp((double)(128 + frac), expo - 133);"),
    "bf16_ties_away": ("    if (rem > 0.5 || (rem == 0.5 && (n & 1)))\n        n += 1;\n    if (n == 256)",
                       "    if (rem >= 0.5)\n        n += 1;\n    if (n == 256)"),
    "bf16_dropped_term": ("for (int64_t k = 0; k < K; ++k)\n        acc += g_lut_bf[arow[k]] * g_lut_bf[brow[k]];",
                          "for (int64_t k = 1; k < K; ++k)\n        acc += g_lut_bf[arow[k]] * g_lut_bf[brow[k]];"),
    "bf16_via_fp32_rounding": ("    return bf16_encode_rne(acc);\n}",
                               "    return bf16_encode_rne((double)(float)acc);\n}"),
    # FP8
    "e4m3_exponent_bias": ("x = e ? ldexp((double)(8 + f), e - 10) : ldexp((double)f, -9);",
                           "x = e ? ldexp((double)(8 + f), e - 11) : ldexp((double)f, -9);"),
    "e4m3_flush_subnormals": ("x = e ? ldexp((double)(8 + f), e - 10) : ldexp((double)f, -9);",
                              "x = e ? ldexp((double)(8 + f), e - 10) : 0.0 * f;"),
    "e4m3_fnuz_nan": ("if (e == 15 && f == 7)\n            return NAN;",
                      "if (v == 0x80)\n            return NAN;"),
    "e5m2_inf_as_max": ("return f ? NAN : (sign ? -INFINITY : INFINITY);",
                        "return f ? NAN : (sign ? -57344.0 : 57344.0);"),
    "fp8_formats_swapped": ("lb[v] = fp8_decode((uint8_t)v, b_e5m2);\n    }\n    int nt = pick_threads(nthreads);\n    const double sc",
                            "lb[v] = fp8_decode((uint8_t)v, a_e5m2);\n    }\n    int nt = pick_threads(nthreads);\n    const double sc"),
    "fp8_cs_formats_swapped": ("lb[v] = fp8_decode((uint8_t)v, b_e5m2);\n    }\n    int nt = pick_threads(nthreads);\n#pragma",
                               "lb[v] = fp8_decode((uint8_t)v, a_e5m2);\n    }\n    int nt = pick_threads(nthreads);\n#pragma"),
    "fp8_round_before_scale": ("D[m * N + n] = f16_encode_rne(sc * acc);",
                               "D[m * N + n] = f16_encode_rne(sc * g_lut[f16_encode_rne(acc)]);"),
    "fp8_dropped_term": ("for (int64_t k = 0; k < K; ++k)\n                acc += la[ar[k]] * lb[br[k]];\n            D[m * N + n] = f16_encode_rne(sc * acc);",
                         "for (int64_t k = 1; k < K; ++k)\n                acc += la[ar[k]] * lb[br[k]];\n            D[m * N + n] = f16_encode_rne(sc * acc);"),
    # FP8 with per-channel weight scales
    "fp8_cs_scale_per_row": ("const float sn = a_scale * b_scale[n];",
                             "const float sn = a_scale * b_scale[m % N];"),
    "fp8_cs_activation_scale_dropped": ("const float sn = a_scale * b_scale[n];",
                                        "const float sn = b_scale[n];"),
    "fp8_cs_round_before_scale": ("D[m * N + n] = f16_encode_rne((double)sn * acc);",
                                  "D[m * N + n] = f16_encode_rne((double)sn * g_lut[f16_encode_rne(acc)]);"),
    # fp16 accumulation
    "acc16_chunk_32": ("        len = 64;\n    }\n    return f16_encode_rne(s);",
                       "        len = 32;\n    }\n    return f16_encode_rne(s);"),
    "acc16_chunks_from_k_start": (
        "int64_t len = K % 64 ? K % 64 : 64;   /* the first chunk */\n    while (k0 < K) {\n        double c = 0.0;\n        for (int64_t k = k0; k < k0 + len; ++k)",
        "int64_t len = 64;   /* the first chunk */\n    while (k0 < K) {\n        double c = 0.0;\n        for (int64_t k = k0; k < k0 + len && k < K; ++k)"),
    "acc16_one_rounding_per_update": ("s = g_lut[f16_encode_rne(s + g_lut[f16_encode_rne(c)])];",
                                      "s = g_lut[f16_encode_rne(s + c)];"),
    "acc16_wide_running_sum": ("s = g_lut[f16_encode_rne(s + g_lut[f16_encode_rne(c)])];",
                               "s = s + c;"),
    "acc16_dropped_first_chunk": ("        s = g_lut[f16_encode_rne(s + g_lut[f16_encode_rne(c)])];\n        k0 += len;",
                                  "        s = k0 ? g_lut[f16_encode_rne(s + g_lut[f16_encode_rne(c)])] : 0.0;\n        k0 += len;"),
    "acc16_wrong_sign": ("            c += g_lut[arow[k]] * g_lut[brow[k]];\n        s = g_lut",
                         "            c -= g_lut[arow[k]] * g_lut[brow[k]];\n        s = g_lut"),
    "acc16_b_row_index": ("out[i] = entry_acc16(A + m * K, B + n * K, K);",
                          "out[i] = entry_acc16(A + m * K, B + ((n + 1) % N) * K, K);"),
}


def _battery():
    """The pin checks, each as a zero-argument callable."""
    return [
        pins.test_p1_decode_exhaustive,
        pins.test_p1_encode_roundtrip_exhaustive,
        pins.test_p1_encode_midpoints_and_neighbours,
        pins.test_p1_encode_overflow_and_random,
        lambda: pins.test_p2a_brute_force_any_finite(K=7, seed=11),
        lambda: pins.test_p2a_brute_force_any_finite(K=17, seed=12),
        lambda: pins.test_p2b_exact_rational(K=33, seed=21),
        pins.test_p3_identity_and_permutation,
        lambda: pins.test_p4_integer_exact((33, 65, 129)),
        lambda: pins.test_p5_all_ones(64),
        pins.test_p5_rank_one,
        pins.test_p6_transpose_symmetry,
        pins.test_p7_ties_and_double_rounding,
        lambda: pins.test_p8_subnormal_inputs(64),
        pins.test_p8_overflow_and_signed_zero_and_empty,
        lambda: epins.test_e1_integer_exact(2.0, -1.0, 7, 9, 13),
        lambda: epins.test_e1_integer_exact(-0.5, 3.0, 33, 17, 64),
        lambda: epins.test_e2_brute_force(3, 31),
        lambda: epins.test_e2_brute_force(16, 32),
        epins.test_e3_zero_product_is_scaled_c_plus_bias,
        epins.test_e4_bias_is_per_column,
        epins.test_e5_reduces_to_plain_and_ignores_c_at_beta_zero,
        bpins.test_b1_decode_exhaustive,
        bpins.test_b2_encode_roundtrip_and_midpoints,
        bpins.test_b2_encode_overflow_and_random,
        lambda: bpins.test_b3_brute_force(8, 61),
        lambda: bpins.test_b3_brute_force(17, 62),
        lambda: bpins.test_b4_integer_exact_then_rounded(33, 20, 300),
        bpins.test_b5_ties_and_double_rounding,
        fpins.test_f1_decode_exhaustive_against_torch,
        fpins.test_f1_decode_defining_constants,
        lambda: fpins.test_f2_brute_force(16, 84, 2.0 ** -7, False),
        lambda: fpins.test_f2_brute_force(33, 85, 0.1, True),
        lambda: fpins.test_f3_integer_exact(33, 20, 256, 0.5, False),
        fpins.test_f4_scale_applied_once_after_the_sum,
        fpins.test_f5_mixed_formats,
        fpins.test_f7_column_scales_reduce_to_per_tensor,
        lambda: fpins.test_f8_column_scales_integer_exact(False),
        lambda: fpins.test_f8_column_scales_integer_exact(True),
        lambda: fpins.test_f9_column_scales_brute_force(7, 131),
        lambda: fpins.test_f9_column_scales_brute_force(24, 132),
        lambda: hpins.test_h1_stall_at_2048(1100, 2048),
        lambda: hpins.test_h1_stall_at_2048(500, 1523),
        hpins.test_h2_chunks_aligned_to_k_end,
        hpins.test_h3_chunk_rounded_before_the_add,
        lambda: hpins.test_h4_one_chunk_is_the_plain_product(33, 41),
        lambda: hpins.test_h4_small_integers_are_exact(200),
        lambda: hpins.test_h5_brute_force_exact(130, 51),
        hpins.test_h5_brute_force_large_sums,
        hpins.test_h6_symmetries,
        hpins.test_h7_empty_overflow_and_sign,
        hpins.test_entries_agree_with_full,
    ]


def _build_mutant(tmp: Path, old: str, new: str) -> Path:
    text = SRC.read_text()
    assert text.count(old) == 1, f"mutation anchor not unique: {old!r}"
    src = tmp / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                           "-std=c11", str(src), "-o", str(lib), "-lm"])
    return lib


def _wrap(path: Path):
    lib = ctypes.CDLL(str(path))
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_f16_decode.argtypes = [p, p, i64]
    lib.oracle_f16_encode.argtypes = [p, p, i64]
    lib.oracle_gemm_nt_f16.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_nt_f16.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_entries.argtypes = [p, p, i64, i64, i64, p, p, i64, p, ctypes.c_int]
    lib.oracle_gemm_nt_f16_entries.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_ex.argtypes = [p, p, p, p, p, i64, i64, i64, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_int]
    lib.oracle_gemm_nt_f16_ex.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_acc16.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_nt_f16_acc16.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_acc16_entries.argtypes = [p, p, i64, i64, i64, p, p, i64, p,
                                                     ctypes.c_int]
    lib.oracle_gemm_nt_f16_acc16_entries.restype = ctypes.c_int
    lib.oracle_bf16_decode.argtypes = [p, p, i64]
    lib.oracle_bf16_encode.argtypes = [p, p, i64]
    lib.oracle_gemm_nt_bf16.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_nt_bf16.restype = ctypes.c_int
    lib.oracle_gemm_nt_bf16_entries.argtypes = [p, p, i64, i64, i64, p, p, i64, p, ctypes.c_int]
    lib.oracle_gemm_nt_bf16_entries.restype = ctypes.c_int
    lib.oracle_fp8_decode.argtypes = [p, p, i64, ctypes.c_int]
    lib.oracle_gemm_nt_fp8.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_int]
    lib.oracle_gemm_nt_fp8.restype = ctypes.c_int
    lib.oracle_gemm_nt_fp8_cs.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_float, p, ctypes.c_int]
    lib.oracle_gemm_nt_fp8_cs.restype = ctypes.c_int
    return lib


def test_unmutated_battery_passes():
    for check in _battery():
        check()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    lib = _wrap(_build_mutant(tmp_path, old, new))
    oracle._load()                      # make sure the real library is not loaded later
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for check in _battery():
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin catches the planted mistake {name!r}"
