"""Plant plausible mistakes in a copy of the oracle and show the pins catch each.

Each mutant is the oracle's C source with one textual change (a dropped term,
a wrong sign, a transposed operand, a wrong rounding rule ...), compiled into
a temporary directory.  The pin checks of ``test_oracle.py`` are run against it
and at least one of them must fail.  This runs on the CPU only; the mistakes
never reach any GPU code.
"""
import os
import sys
import tempfile

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import test_oracle as T  # noqa: E402

import oracle  # noqa: E402

MUTANTS = {
    "drop_last_k_term": [("k < K; ++k", "k < K - 1; ++k")],
    "silu_sign_flipped": [("g / (1.0f + expf(-g))", "g / (1.0f + expf(g))")],
    "silu_is_sigmoid": [("g / (1.0f + expf(-g))", "1.0f / (1.0f + expf(-g))")],
    "gate_up_swapped": [("oracle_silu(g[j]);\n                    const float p = s * u[j];",
                         "oracle_silu(u[j]);\n                    const float p = s * g[j];")],
    "round_truncate": [("b += 0x7FFFu + lsb;", "b += 0u * lsb;")],
    "round_ties_away": [("b += 0x7FFFu + lsb;", "b += 0x8000u + 0u * lsb;")],
    "nan_not_quieted": [("(b >> 16) | 0x0040u", "(b >> 16)")],
    "weight_column_reversed": [("bf16_to_f32(w1[j])", "bf16_to_f32(w1[N - 1 - j])")],
    "activation_transposed": [("A[i * K + k]", "A[k * M + i]")],
    "decode_shift_wrong": [("(uint32_t)h << 16", "(uint32_t)h << 15")],
    "up_uses_w1": [("bf16_to_f32(w2[j])", "bf16_to_f32(w1[j])")],
    "output_transposed": [("Y[i * N + j] = oracle_bf16_rne(p);", "Y[j * M + i] = oracle_bf16_rne(p);")],
    "sum_decreasing_k": [("for (int64_t k = 0; k < K; ++k) {\n                    const float a",
                          "for (int64_t k = K - 1; k >= 0; --k) {\n                    const float a"),
                         ("for (int64_t k = 0; k < K; ++k) {\n            const float a",
                          "for (int64_t k = K - 1; k >= 0; --k) {\n            const float a")],
    "unfused_skips_gate_rounding": [("oracle_silu(bf16_to_f32(Gb[t]))",
                                     "oracle_silu(bf16_to_f32(Gb[t]) + 0x1p-9f * bf16_to_f32(Gb[t]))")],
    # FP8 variant
    "e4m3_exponent_bias_8": [("e - 7 - 3", "e - 8 - 3")],
    "e4m3_subnormal_scale": [("ldexpf((float)m, -9)", "ldexpf((float)m, -10)")],
    "e4m3_nan_codes_wrong": [("e == 15 && m == 7", "e == 15")],
    "fp8_scales_swapped": [("const float G = g[j] * sg;\n                    const float U = u[j] * su;",
                            "const float G = g[j] * su;\n                    const float U = u[j] * sg;")],
    "fp8_up_scale_dropped": [("const float U = u[j] * su;", "const float U = u[j];")],
    "fp8_gate_uses_w2": [("const float pg = a * table[w1[j]];", "const float pg = a * table[w2[j]];")],
}

CHECKS = [
    ("rne_table", lambda o: T.check_rne_table(o)),
    ("rne_vs_torch", lambda o: T.check_rne_vs_torch(o, n=20000)),
    ("nan", lambda o: T.test_rne_nan_never_inf(o)),
    ("silu", lambda o: T.check_silu_closed_forms(o)),
    ("bruteforce", lambda o: T.check_bruteforce(
        o, [(m, k, n) for m in (1, 3, 7) for k in (1, 8, 100) for n in (1, 7, 33)])),
    ("order", lambda o: T.test_accumulation_order_is_increasing_k(o)),
    ("integer", lambda o: T.check_integer_regime(o)),
    ("invariants", lambda o: T.check_invariants(o)),
    ("unfused", lambda o: T.check_unfused(o)),
    ("e4m3", lambda o: T.test_e4m3_decode_matches_library(o)),
    ("fp8_bound", lambda o: T.test_fp8_bruteforce_bound(o)),
    ("fp8_exact", lambda o: T.test_fp8_exact_regime(o)),
    ("fp8_invariants", lambda o: T.test_fp8_scale_and_zero_invariants(o)),
]


def build_mutant(name, edits, tmpdir):
    src = open(oracle.SOURCE).read()
    for old, new in edits:
        assert old in src, "mutation %s: pattern not found: %r" % (name, old)
        src = src.replace(old, new)
    path = os.path.join(tmpdir, "oracle_%s.c" % name)
    with open(path, "w") as fh:
        fh.write(src)
    lib = oracle.compile_source(path, os.path.join(tmpdir, "liboracle_%s.so" % name))
    return oracle.Oracle(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    with tempfile.TemporaryDirectory() as d:
        mut = build_mutant(name, MUTANTS[name], d)
        caught = []
        for cname, fn in CHECKS:
            try:
                fn(mut)
            except (AssertionError, ValueError, RuntimeError):
                caught.append(cname)
        assert caught, "mutant %s survived every pin" % name


def test_unmutated_copy_passes_every_pin():
    with tempfile.TemporaryDirectory() as d:
        ok = build_mutant("none", [], d)
        for cname, fn in CHECKS:
            fn(ok)
