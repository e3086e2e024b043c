"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one of them.

Each mutant is a textual edit of oracle/mma_oracle.c compiled into a
temporary library; the original is never touched.  The battery run against
each mutant uses only the page-derived and mathematical pins of
test_oracle_pins.py (hand-derived values, neutral subgroups, library casts,
the exact-integer closed form, IEEE special values, invariants) -- not the
rational model.
"""
import os
import shutil

import numpy as np
import pytest

import oracle
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "mma_oracle.c")

MUTANTS = {
    "ampere_width_22": [("g1 = group_sum(T1, 9, 23);", "g1 = group_sum(T1, 9, 22);")],
    "ampere_stage2_width_22": [("g2 = group_sum(T2, 9, 23);", "g2 = group_sum(T2, 9, 22);")],
    "hopper_width_23": [("g = group_sum(T, 17, 24);", "g = group_sum(T, 17, 23);")],
    "stage1_norm_25_bits": [("S1 = norm(g1, 23, 24);", "S1 = norm(g1, 23, 25);")],
    "alignment_rounds_half_up": [
        ("A = shift_right_truncating(M, emax - T[i].E);",
         "A = shift_right_truncating(M + ((emax - T[i].E) > 0 && (emax - T[i].E) < 62 ? "
         "((int64_t)1 << (emax - T[i].E - 1)) : 0), emax - T[i].E);")],
    "floor_not_truncate": [
        ("S += T[i].s ? -A : A;",
         "S += T[i].s ? -(shift_right_truncating(M + (((int64_t)1 << ((emax - T[i].E) < 62 ? "
         "(emax - T[i].E) : 62)) - 1), emax - T[i].E)) : A;")],
    "sign_dropped": [("S += T[i].s ? -A : A;", "S += A;")],
    "stage2_drops_last_product": [("g2 = group_sum(T2, 9, 23);", "g2 = group_sum(T2, 8, 23);")],
    "hopper_drops_C": [("g = group_sum(T, 17, 24);", "g = group_sum(T + 1, 16, 24);")],
    "stages_swapped": [("T1[1 + k] = P[k];", "T1[1 + k] = P[8 + k];"),
                       ("T2[1 + k] = P[8 + k];", "T2[1 + k] = P[k];")],
    "products_normalised": [
        ("    p.m = a.m * b.m;\n",
         "    p.m = a.m * b.m;\n    if (p.m >= ((int64_t)1 << (p.f + 1))) { p.E += 1; p.f += 1; }\n")],
    "subnormal_renormalised": [
        ("    r.kind = (frac == 0) ? K_ZERO : K_FINITE;\n    return r;",
         "    r.kind = (frac == 0) ? K_ZERO : K_FINITE;\n"
         "    while (r.m != 0 && r.m < ((int64_t)1 << fm->frac_bits)) { r.m <<= 1; r.E -= 1; }\n"
         "    return r;")],
    "zeros_join_max_search": [
        ("    if (T[i].kind == K_FINITE) {\n      if (!have",
         "    if (T[i].kind == K_FINITE || T[i].kind == K_ZERO) {\n      if (!have")],
    "writeback_rounds_half_up": [
        ("int64_t m24 = (n > 24) ? (mag >> (n - 24)) : (mag << (24 - n));",
         "int64_t m24 = (n > 24) ? ((mag + ((int64_t)1 << (n - 25))) >> (n - 24)) : (mag << (24 - n));")],
    "overflow_saturates": [("if (L >= 128) return sign | 0x7F800000u;",
                            "if (L >= 128) return sign | 0x7F7FFFFFu;")],
    "B_transposed": [("b[k] = load_code(j->B, j->dtype, (16 * t + k) * j->N + col);",
                      "b[k] = load_code(j->B, j->dtype, col * j->K + 16 * t + k);")],
    "chain_not_carried": [("        c = mma_step(j->model, fm, c, a, b);\n      }\n      j->D",
                           "        c = mma_step(j->model, fm, t == 0 ? c : 0u, a, b);\n      }\n      j->D")],
    "C_sign_ignored": [("  term C = decode(&FMT_FP32, c);", "  term C = decode(&FMT_FP32, c & 0x7FFFFFFFu);")],
    "e4m3_nan_as_finite": [("  if (fm->fn_nan && ef == emask && frac == fmask) {",
                            "  if (0) {")],
    "cancellation_gives_minus_zero": [("  g.zero_sign = 0; /* exact cancellation gives +0 */",
                                       "  g.zero_sign = 1;")],
    "inf_times_zero_is_zero": [("(a.kind == K_ZERO && b.kind == K_INF)) {\n    p.kind = K_NAN;",
                                "(a.kind == K_ZERO && b.kind == K_INF)) {\n    p.kind = K_ZERO;")],
    "opposite_infs_give_inf": [("if (any_nan || (pos_inf && neg_inf)) return CANONICAL_NAN;",
                                "if (any_nan) return CANONICAL_NAN;")],
    "nan_C_ignored": [("  if (C.kind == K_NAN) any_nan = 1;\n", "")],
}


def _battery(orc):
    """Return the name of the first pin that fails, or None."""
    for case in P.PINS:
        try:
            _golden(orc, case)
        except AssertionError:
            return "golden:" + case["name"]
    if P._neutral_sets(orc, "ampere") != {tuple(range(9)), tuple(range(17))}:
        return "neutral:ampere"
    if P._neutral_sets(orc, "hopper") != {tuple(range(17))}:
        return "neutral:hopper"
    checks = [
        ("single:fp16", lambda: P.test_single_term_fp16_all_codes(orc, "ampere")),
        ("single:bf16", lambda: P.test_single_term_bf16_all_codes(orc, "hopper")),
        ("single:e4m3", lambda: P.test_single_term_e4m3_all_codes(orc)),
        ("e4m3_pairs", lambda: P.test_e4m3_all_products_exact(orc)),
        ("bf16_pairs", lambda: P.test_bf16_random_products_exact_or_inf(orc, "hopper")),
    ]
    for model, dt in [("ampere", "fp16"), ("hopper", "fp16"), ("ampere", "bf16"),
                      ("hopper", "e4m3")]:
        checks.append((f"closed_form:{model}:{dt}",
                       lambda m=model, d=dt: P.test_integer_gemm_closed_form(orc, m, d)))
    for model, dt in [(0, 0), (1, 1)]:
        checks.append((f"sign_symmetry:{model}:{dt}",
                       lambda m=model, d=dt: P.test_sign_symmetry(orc, m, d)))
        checks.append((f"permutation:{model}:{dt}",
                       lambda m=model, d=dt: P.test_permutation_within_groups(orc, m, d)))
    checks.append(("zero_sign", lambda: _zero_sign(orc)))
    for case in P.SPECIAL_CASES:
        checks.append(("special:" + case[0],
                       lambda c=case: P.test_special_values_follow_ieee(orc, c)))
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            return name
    return None


def _golden(orc, case):
    a, b, c = P._slots_to_dot(case)
    for model, want in case["expect"].items():
        got = int(orc.dots(model, case["dtype"], a, b, c)[0])
        assert got == int(want, 16)


def _zero_sign(orc):
    """Exact cancellation of two products gives +0 (IEEE addition toward
    zero); a sum of only -0 terms gives -0."""
    a = np.zeros((2, 16), np.uint16)
    b = np.zeros((2, 16), np.uint16)
    a[0, 0], b[0, 0], a[0, 1], b[0, 1] = 0x3C00, 0x3C00, 0xBC00, 0x3C00
    a[1, :] = 0x8000
    b[1, :] = 0x3C00
    c = np.array([0, 0x80000000], np.uint32)
    for model in ("ampere", "hopper"):
        d = orc.dots(model, "fp16", a, b, c)
        assert d[0] == 0 and d[1] == 0x80000000


def test_unmutated_copy_passes(tmp_path):
    src = tmp_path / "orig.c"
    shutil.copy(SRC, src)
    lib = oracle.build_library(str(src), str(tmp_path / "orig.so"))
    assert _battery(lib) is None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    text = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
        text = text.replace(old, new)
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = oracle.build_library(str(src), str(tmp_path / f"{name}.so"))
    caught_by = _battery(lib)
    assert caught_by is not None, f"mutant {name} survived every pin"
