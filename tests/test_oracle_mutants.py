"""Mutation check of the oracle's pins (CPU).

Each mutant is a copy of oracle.cpp with one plausible mistake planted by an
exact text edit (a dropped or wrong term, a wrong sign, index or rounding
rule). It is compiled on its own and the oracle pin tests run against it in a
subprocess; every mutant must be killed (pytest exits 1). The identity mutant
(no edit) must survive, which shows that the injection itself is sound. This
follows the mutation-matrix scheme of "mmaemu testing" (T4: identity mutants
survive, a sign flip is killed), applied to this repository's oracle.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")
PINS = [os.path.join(ROOT, "tests", "test_oracle_fp8.py"), os.path.join(ROOT, "tests", "test_oracle_gemm.py"),
        os.path.join(ROOT, "tests", "test_oracle_atom.py"), os.path.join(ROOT, "tests", "test_oracle_fp4.py"),
        os.path.join(ROOT, "tests", "test_oracle_grouped.py"),
        os.path.join(ROOT, "tests", "test_oracle_grouped_layouts.py")]

# name -> (old text, new text); old text must occur exactly once
MUTANTS = {
    "identity": None,
    "control_sign_flip": ("                        S += t;\n                        T += std::fabs(t);\n                    }\n                    const double s",
                          "                        S -= t;\n                        T += std::fabs(t);\n                    }\n                    const double s"),
    "round_truncates": ("double r = std::nearbyint(ax / q) * q;", "double r = std::trunc(ax / q) * q;"),
    "round_ties_away": ("double r = std::nearbyint(ax / q) * q;", "double r = std::round(ax / q) * q;"),
    "no_saturation": ("if (f.saturate) r = f.maxv;", "if (false) r = f.maxv;"),
    "e4m3_subnormal_exp": ("std::ldexp((double)m, -9)", "std::ldexp((double)m, -10)"),
    "e5m2_bias": ("std::ldexp((double)(4 + m), e - 17)", "std::ldexp((double)(4 + m), e - 16)"),
    "e4m3_nan_code": ("if (e == 15 && m == 7) return std::nan(\"\");", "if (e == 15 && m == 6) return std::nan(\"\");"),
    "block_scale_index": ("const double ah = Am[k] * sa_at(m, k / 128);", "const double ah = Am[k] * sa_at(m, k / 64 % KB);"),
    "scale_b_128_rows": ("scale_b[(n / 128) * KB + kb]", "scale_b[(n % 128) * KB + kb]"),
    "float_accumulator": ("                    double S = +0.0, T = 0.0;\n                    for (int64_t k = 0; k < K; ++k) {\n                        const double t = Am[k] * Bn[k];",
                          "                    float S = +0.0f; double T = 0.0;\n                    for (int64_t k = 0; k < K; ++k) {\n                        const double t = Am[k] * Bn[k];"),
    "chunk_partial_not_rounded": ("const float part = to_f32(P);", "const double part = P;"),
    "scale_result_ignored": ("    v *= sr;\n", "    v *= 1.0;\n"),
    "amax_tie_last": ("(av == best && idx < best_idx)", "(av == best && idx > best_idx)"),
    "sf_group_index": ("(double)sfa[(l * M + m) * KS + k / sf_vec];", "(double)sfa[(l * M + m) * KS + k / (2 * sf_vec)];"),
    "nan_not_canonical": ("if (std::isnan(r)) return f.nan_bits;", "if (std::isnan(r)) return f.nan_bits - 1;"),
    "bias_dropped": ("if (bias) v = accum == ORC_ACC_EXACT ? v + bias[n] : (double)to_f32(v + bias[n]);",
                     "if (bias) v = v;"),
    "bias_exact_rounded_f32": ("if (bias) v = accum == ORC_ACC_EXACT ? v + bias[n] : (double)to_f32(v + bias[n]);",
                               "if (bias) v = (double)to_f32(v + bias[n]);"),
    "e8m0_bias": ("std::ldexp(1.0, (int)e - 127)", "std::ldexp(1.0, (int)e - 126)"),
    "e8m0_nan_code": ("if (e == 0xFF) return std::nan(\"\");", "if (e == 0xFE) return std::nan(\"\");"),
    "atom_storage_inner_swapped": ("* 32 + i0) * 4 + i1) * 4 + j0;", "* 32 + i0) * 4 + j0) * 4 + i1;"),
    "atom_rows_i1_fastest": ("const int64_t mn = i0 + 32 * i1 + 128 * i2;", "const int64_t mn = 4 * i0 + i1 + 128 * i2;"),
    "atom_block_order": ("((((l * MB + i2) * KB + j1) * 32", "((((l * KB + j1) * MB + i2) * 32"),
    "e2m1_bias": ("std::ldexp((double)(2 + m), e - 2)", "std::ldexp((double)(2 + m), e - 1)"),
    "e2m1_subnormal": ("std::ldexp((double)m, -1)", "std::ldexp((double)m, 0)"),
    "fp4_sign_dropped": ("(row[k >> 1] >> (4 * (k & 1))) & 15", "(row[k >> 1] >> (4 * (k & 1))) & 7"),
    "group_b_operand": ("b + g * stride_b, b_fmt", "b + (g / 2) * stride_b, b_fmt"),
    "group_a_rows": ("a + r0 * lda, a_fmt", "a + (r0 / 2) * lda, a_fmt"),
    "group_output_rows": ("value ? value + r0 * N : nullptr", "value ? value + (r0 / 2) * N : nullptr"),
    "group_row_count_unchecked": ("    if (next != batch_sum) return ORC_ERR_ARG;\n    const int width",
                                  "    if (false) return ORC_ERR_ARG;\n    const int width"),
    "e2m1_out_max": ("{1, 1, 4, 6.0, false, true, 0x7u}", "{1, 1, 4, 4.0, false, true, 0x7u}"),
    "e2m1_c_high_nibble_first": ("*cb = (n & 1) ? (uint8_t)((*cb & 0x0F) | (code << 4)) : code;",
                                 "*cb = (n & 1) ? (uint8_t)((*cb & 0xF0) | code) : (uint8_t)(code << 4);"),
    "zero_chain_negative": ("double S = +0.0, T = 0.0;\n                    for (int64_t k = 0; k < K; ++k) {\n                        const double t = Am[k] * Bn[k];\n                        S += t;",
                            "double S = -0.0, T = 0.0;\n                    for (int64_t k = 0; k < K; ++k) {\n                        const double t = Am[k] * Bn[k];\n                        S += t;"),
}


def _run_mutant(name, edit, workdir):
    src = open(SRC).read()
    if edit is not None:
        old, new = edit
        assert src.count(old) == 1, f"{name}: pattern occurs {src.count(old)} times"
        src = src.replace(old, new)
    d = os.path.join(workdir, name)
    os.makedirs(d)
    cpp = os.path.join(d, "oracle.cpp")
    lib = os.path.join(d, "liboracle.so")
    open(cpp, "w").write(src)
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    "-o", lib, cpp], check=True)
    env = dict(os.environ, ORACLE_LIB_PATH=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


def test_every_mutant_is_killed_and_identity_survives():
    work = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda kv: _run_mutant(kv[0], kv[1], work), MUTANTS.items()))
    finally:
        shutil.rmtree(work, ignore_errors=True)
    problems = []
    for name, rc, out in results:
        if name == "identity":
            if rc != 0:
                problems.append(f"identity mutant did not survive (rc={rc}):\n{out}")
        elif rc != 1:
            problems.append(f"mutant {name} survived (rc={rc})")
    assert not problems, "\n".join(problems)
