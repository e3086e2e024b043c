"""The characterisation harness (bit_exact_matrix_amd.characterise) pointed
at the oracle: it must recover the pages' Target Tests results for every
model and format, and each probe must report the behaviour a planted oracle
mistake gives it (so that no probe passes vacuously)."""
import json
import os

import pytest

import oracle
from bit_exact_matrix_amd import characterise as ch

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = json.load(open(os.path.join(HERE, "golden", "target_tests.json")))["models"]
COMBOS = [("ampere", "fp16"), ("hopper", "fp16"), ("ampere", "bf16"), ("hopper", "bf16"),
          ("hopper", "e4m3"), ("lovelace", "fp16")]


def oracle_dots(model, dtype, lib=None):
    return lambda a, b, c: oracle.dots(model, dtype, a, b, c, lib=lib)


@pytest.mark.parametrize("model,dtype", COMBOS)
def test_recovers_the_target_tests_table(orc, model, dtype):
    got = ch.characterise(oracle_dots(model, dtype), dtype)
    want = TABLE[model]
    for key in want:
        assert got[key] == want[key], (model, dtype, key, got[key])


# internal widths changed consistently (group grids, stage-1 width and
# write-back together; the oracle needs F >= 23 to hold C exactly)
WIDTH_MUTANTS = {
    "ampere_25_bits": [("g1 = group_sum(T1, 9, 23);", "g1 = group_sum(T1, 9, 24);"),
                       ("S1 = norm(g1, 23, 24);", "S1 = norm(g1, 24, 25);"),
                       ("g2 = group_sum(T2, 9, 23);", "g2 = group_sum(T2, 9, 24);"),
                       ("return writeback_fp32(g2, 23);", "return writeback_fp32(g2, 24);")],
    "hopper_24_bits": [("g = group_sum(T, 17, 24);", "g = group_sum(T, 17, 23);"),
                       ("return writeback_fp32(g, 24);", "return writeback_fp32(g, 23);")],
}

# mutant of the oracle source -> (model, dtype, probe result key, expected value)
PLANTED = {
    "ampere_25_bits": ("ampere", "fp16", "internal_width", 25),
    "hopper_24_bits": ("hopper", "bf16", "internal_width", 24),
    "ampere_width_22": ("ampere", "fp16", "internal_width", None),   # inconsistent scaling
    "alignment_rounds_half_up": ("ampere", "fp16", "alignment_rounding", "nearest"),
    "floor_not_truncate": ("hopper", "fp16", "alignment_rounding", "down"),
    "products_normalised": ("ampere", "bf16", "product_normalisation", "normalised first"),
    "subnormal_renormalised": ("hopper", "e4m3", "subnormal_products", "renormalised"),
    "stages_swapped": ("ampere", "fp16", "groups",
                       [[0, 9, 10, 11, 12, 13, 14, 15, 16], [1, 2, 3, 4, 5, 6, 7, 8]]),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_probe_reports_a_planted_behaviour(tmp_path, name):
    from test_oracle_mutants import MUTANTS
    text = open(oracle.SRC).read()
    for old, new in {**MUTANTS, **WIDTH_MUTANTS}[name]:
        assert old in text, f"mutant anchor missing: {old!r}"
        text = text.replace(old, new)
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = oracle.build_library(str(src), str(tmp_path / f"{name}.so")).lib
    model, dtype, key, want = PLANTED[name]
    got = ch.characterise(oracle_dots(model, dtype, lib), dtype, neutral=(key == "groups"))
    assert got[key] == want, (name, got[key])


def test_exact_encoders():
    from fractions import Fraction
    assert ch.code_of("fp16", 1) == 0x3C00
    assert ch.code_of("bf16", -2) == 0xC000
    assert ch.code_of("e4m3", Fraction(1, 512)) == 0x01      # smallest subnormal
    assert ch.code_of("e4m3", 448) == 0x7E
    with pytest.raises(ValueError):
        ch.code_of("e4m3", 512)
    a, b = ch.factor("fp16", Fraction(3, 2) * Fraction(1, 1 << 24))
    va = {v: c for v, c in ch._finite_values("fp16").items()}
    inv = {c: v for v, c in va.items()}
    assert inv[a] * inv[b] == Fraction(3, 2) * Fraction(1, 1 << 24)
    assert ch.f32_bits(Fraction(1)) == 0x3F800000
    with pytest.raises(ValueError):
        ch.f32_bits(Fraction(1, 3))
