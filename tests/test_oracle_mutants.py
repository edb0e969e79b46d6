"""Plant plausible mistakes in a copy of the oracle and check that the pins fail.

Each mutant is oracle.c with one textual change (a dropped term, a wrong scale,
sign or index, a transposed operand, a fused multiply-add, a reversed band
order, a missing special case).  It is compiled into a temporary library and
the fast pins run against it in a subprocess; the subprocess must fail.  The
unmodified oracle must pass the same selection.  CPU only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

FAST_PINS = ("test_split_golden or test_split_rne_golden or test_emu_identity or test_emu_recombination or "
             "test_naive_f32 or test_gemm_f64_small_integers or test_gemm_f64_vs_numpy or "
             "test_emu_tolerance or test_emu_three_product or test_emu_band_drop or "
             "test_emu_small_integers or test_emu_special or test_gelu or test_emu_scaled_permutation")

MUTANTS = {
    "split_x0_round_nearest": ("mode == ORC_SPLIT_RNE_MODE ? rne_bf16(x) : trunc_bf16(x);",
                               "mode == ORC_SPLIT_RNE_MODE ? rne_bf16(x) : (uint16_t)((bits_of(x) + 0x8000u) >> 16);"),
    "rne_ties_away": ("return (lo & 1u) ? hi : lo;", "return hi;"),
    "rne_nearest_by_bits": ("if (dl < dh) return lo;", "if (bits_of(v) & 0x8000u) return hi; if (1) return lo;"),
    "rne_x1_truncated": ("mode == ORC_SPLIT_RNE_MODE ? rne_bf16(tf) : trunc_bf16(tf);", "trunc_bf16(tf);"),
    "split_scale_2^7": ("double t = r * 256.0;", "double t = r * 128.0;"),
    "split_x2_unscaled": ("double s = (t - (double)bf16_value(h1)) * 256.0;",
                          "double s = (t - (double)bf16_value(h1)) * 1.0;"),
    "split_no_nan_quiet": ("if (u & 0x007FFFFFu) hi |= 0x0040u;", ";"),
    "split_no_inf_case": ("if ((u & 0x7F800000u) == 0x7F800000u) {", "if (0) {"),
    "emu_drop_a2b0": ("if (s >= nbands) continue;", "if (s >= nbands || (p == 2 && q == 0)) continue;"),
    "emu_band2_weight": ("acc = fmaf(S[2 * N + j], 0x1p-16f, acc);", "acc = fmaf(S[2 * N + j], 0x1p-15f, acc);"),
    "emu_sign_s0": ("C[r * ldc + j] = acc + S[j];", "C[r * ldc + j] = acc - S[j];"),
    "emu_transposed_b": ("orc_split_one_mode(B[k * ldb + j], smode, &h[0], &h[1], &h[2]);",
                         "orc_split_one_mode(B[j * ldb + k], smode, &h[0], &h[1], &h[2]);"),
    "emu_largest_band_first": (
        "float acc = 0x1p-32f * S[4 * N + j];\n"
        "            acc = fmaf(S[3 * N + j], 0x1p-24f, acc);\n"
        "            acc = fmaf(S[2 * N + j], 0x1p-16f, acc);\n"
        "            acc = fmaf(S[1 * N + j], 0x1p-8f, acc);\n"
        "            C[r * ldc + j] = acc + S[j];",
        "float acc = S[j];\n"
        "            acc = fmaf(S[1 * N + j], 0x1p-8f, acc);\n"
        "            acc = fmaf(S[2 * N + j], 0x1p-16f, acc);\n"
        "            acc = fmaf(S[3 * N + j], 0x1p-24f, acc);\n"
        "            C[r * ldc + j] = fmaf(S[4 * N + j], 0x1p-32f, acc);"),
    "f64_reversed_column": ("for (int64_t j = 0; j < N; ++j) c[j] += a * (double)b[j];",
                            "for (int64_t j = 0; j < N; ++j) c[j] += a * (double)b[N - 1 - j];"),
    "f64_signed_g": ("g[j] += fabs(a * (double)b[j]);", "g[j] += a * (double)b[j];"),
    "naive_fma": ("float p = a * b[j];\n                c[j] = c[j] + p;", "c[j] = fmaf(a, b[j], c[j]);"),
    "trunc_band1_weight": ("static const double weight[5] = {1.0, 0x1p-8, 0x1p-16, 0x1p-24, 0x1p-32};",
                           "static const double weight[5] = {1.0, 0x1p-7, 0x1p-16, 0x1p-24, 0x1p-32};"),
    "gelu_half_scale": ("y[i] = (float)(0.5 * x[i]", "y[i] = (float)(0.25 * x[i]"),
}


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-fPIC", "-shared", "-o", str(lib), str(src), "-lm"], check=True)
    return str(lib)


def _run_pins(lib):
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", FAST_PINS, os.path.join(ROOT, "tests", "test_oracle_split.py"),
           os.path.join(ROOT, "tests", "test_oracle_gemm.py")]
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)


def test_unmodified_oracle_passes_fast_pins(tmp_path):
    r = _run_pins(_build(tmp_path, "orig", open(SRC).read()))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    r = _run_pins(_build(tmp_path, name, text.replace(old, new)))
    assert r.returncode != 0, f"mutant {name} passed every fast pin"
