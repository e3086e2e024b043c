"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
hand-derived values from the pages' worked facts (tests/golden/pins.json),
library casts (numpy float16, bfloat16 as a 16-bit shift, torch
float8_e4m3fn), exact integer arithmetic, the neutral-subgroup structure the
pages report, invariants of the model, and an independent exact-rational
restatement of the rules (tests/rational_model.py).
"""
import json
import os

import numpy as np
import pytest

import rational_model as RM

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = json.load(open(os.path.join(HERE, "golden", "pins.json")))["cases"]
DT = {"fp16": 0, "bf16": 1, "e4m3": 2}
MODEL = {"ampere": 0, "hopper": 1}


def _slots_to_dot(case):
    d = DT[case["dtype"]]
    cd = np.uint8 if d == 2 else np.uint16
    a = np.zeros((1, 16), cd)
    b = np.zeros((1, 16), cd)
    for k, ac, bc in case["slots"]:
        a[0, k] = int(ac, 16)
        b[0, k] = int(bc, 16)
    c = np.array([int(case["c"], 16)], np.uint32)
    return a, b, c


@pytest.mark.parametrize("case", PINS, ids=[c["name"] for c in PINS])
def test_golden_pin(orc, case):
    a, b, c = _slots_to_dot(case)
    for model, want in case["expect"].items():
        got = int(orc.dots(model, case["dtype"], a, b, c)[0])
        assert got == int(want, 16), f"{case['name']} {model}: {got:#010x} != {want}"
        rm = RM.step(MODEL[model], DT[case["dtype"]], int(c[0]),
                     [int(x) for x in a[0]], [int(x) for x in b[0]])
        assert rm == int(want, 16), f"rational model {case['name']} {model}: {rm:#010x}"
        for why, bad in case["wrong"].items():
            assert got != int(bad, 16) or bad == want


# ------------------------------------------------ neutral subgroups (Alg. 4)
def _neutral_sets(orc, model):
    """Enumerate every subset S of {C, P1..P16} with |S| >= 2.  Engineered:
    S's terms are huge (2^24) and cancel exactly (pairs x, -x; a triple x, x,
    -2x for an odd count without C; C = -x for an odd count with C); every
    slot outside S holds a small non-zero term with low-order bits.  Zeroed:
    S's A entries (and C) are +0.  S is neutral iff both give the same bits."""
    big_a, big_b = 0x7000, 0x7000          # 2^12 * 2^12 = 2^24
    big_a2 = 0x7400                        # 2^13: product 2^25 = 2 * 2^24
    small_a, small_b = 0x3C01, 0x3C01      # (1 + 2^-10)^2
    c_small = 0x3F800001
    subsets = []
    a_eng, b_eng, c_eng, a_zer, b_zer, c_zer = [], [], [], [], [], []
    for mask in range(1 << 17):
        members = [i for i in range(17) if mask >> i & 1]
        if len(members) < 2:
            continue
        has_c = 0 in members
        prods = [i - 1 for i in members if i > 0]
        a = np.full(16, small_a, np.uint16)
        b = np.full(16, small_b, np.uint16)
        c = c_small
        signs = []
        n = len(prods)
        if has_c:
            signs = [(+1 if j % 2 == 0 else -1) for j in range(n)]
            for j, k in enumerate(prods):
                a[k] = big_a | (0x8000 if signs[j] < 0 else 0)
                b[k] = big_b
            total = sum(signs)
            c = 0x4B800000 if total < 0 else (0xCB800000 if total > 0 else 0)  # +-2^24
        else:
            for k in prods:
                a[k], b[k] = big_a, big_b
            if n % 2 == 0:
                for j, k in enumerate(prods):
                    if j % 2:
                        a[k] |= 0x8000
            else:  # x + x - 2x, then pairs
                a[prods[2]] = big_a2 | 0x8000
                for j, k in enumerate(prods[3:]):
                    if j % 2:
                        a[k] |= 0x8000
        a_eng.append(a)
        b_eng.append(b)
        c_eng.append(c)
        az = a.copy()
        for k in prods:
            az[k] = 0
        a_zer.append(az)
        b_zer.append(b.copy())
        c_zer.append(0 if has_c else c)
        subsets.append(tuple(members))
    A1, B1, C1 = np.array(a_eng), np.array(b_eng), np.array(c_eng, np.uint32)
    A2, B2, C2 = np.array(a_zer), np.array(b_zer), np.array(c_zer, np.uint32)
    d1 = orc.dots(model, "fp16", A1, B1, C1)
    d2 = orc.dots(model, "fp16", A2, B2, C2)
    return {s for s, x, y in zip(subsets, d1, d2) if x == y}


def test_neutral_subgroups_ampere(orc):
    full = tuple(range(17))
    assert _neutral_sets(orc, "ampere") == {tuple(range(9)), full}


def test_neutral_subgroups_hopper(orc):
    assert _neutral_sets(orc, "hopper") == {tuple(range(17))}


def test_neutral_subgroups_lovelace(orc):
    """Lovelace has Ampere's structure ("Recovered Ampere FP16 pipeline"):
    the neutral-subgroup characterisation must find Ampere's two groups."""
    assert _neutral_sets(orc, "lovelace") == {tuple(range(9)), tuple(range(17))}


def test_lovelace_is_rejected_with_e4m3(orc):
    a = np.zeros((1, 16), np.uint8)
    with pytest.raises(ValueError):
        orc.dots("lovelace", "e4m3", a, a, np.zeros(1, np.uint32))


# ------------------------------------------------ single-term library casts
def _single_term(orc, model, dtype, codes, one):
    """D = c + a*1 with every other product -0 and C = -0: D = float32(a)."""
    n = len(codes)
    cd = np.uint8 if dtype == "e4m3" else np.uint16
    neg_zero = 0x80 if dtype == "e4m3" else 0x8000
    a = np.full((n, 16), neg_zero, cd)
    b = np.full((n, 16), one, cd)
    a[:, 0] = codes
    c = np.full(n, 0x80000000, np.uint32)
    return orc.dots(model, dtype, a, b, c)


def _assert_same_or_nan(got, ref_f32):
    ref = ref_f32.view(np.uint32)
    isnan = np.isnan(ref_f32)
    assert np.all(got[isnan] == 0x7FC00000)
    bad = np.nonzero((got != ref) & ~isnan)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first index {bad[:5]}"


# ------------------------------------------------ special values by IEEE 754
NAN32, PINF32, NINF32 = 0x7FC00000, 0x7F800000, 0xFF800000
_F16 = {"inf": 0x7C00, "-inf": 0xFC00, "nan": 0x7E00, "1": 0x3C00, "-1": 0xBC00,
        "2": 0x4000, "max": 0x7BFF, "0": 0x0000, "-0": 0x8000}
# (name, dtype, C word, {k: (a, b)}, D word); unlisted slots are +0 * +0.
# Each D follows from IEEE 754 alone: inf*0 is invalid, inf + (-inf) is
# invalid, NaN propagates (reading O12: as the canonical quiet NaN), inf
# absorbs any finite sum.  Ampere gives the same word as Hopper: the two
# stages see the same inf/NaN set between them.
SPECIAL_CASES = [
    ("inf_times_zero", "fp16", 0, {0: ("inf", "0")}, NAN32),
    ("minus_zero_times_minus_inf_stage2", "fp16", 0, {9: ("-0", "-inf")}, NAN32),
    ("opposite_infs_across_stages", "fp16", 0, {0: ("inf", "1"), 15: ("-inf", "1")}, NAN32),
    ("inf_product_against_minus_inf_C", "fp16", NINF32, {3: ("inf", "1")}, NAN32),
    ("nan_C_with_payload", "fp16", 0x7FC00001, {0: ("1", "1")}, NAN32),
    ("nan_C_negative", "fp16", 0xFFC00000, {}, NAN32),
    ("inf_C_absorbs_largest_sum", "fp16", PINF32, {k: ("max", "max") for k in range(16)},
     PINF32),
    ("minus_inf_product_absorbs_sum", "fp16", 0,
     {**{k: ("max", "max") for k in range(16)}, 5: ("-inf", "2")}, NINF32),
    ("minus_inf_C_absorbs_sum", "fp16", NINF32, {k: ("max", "max") for k in range(16)},
     NINF32),
    ("inf_times_inf", "fp16", 0, {0: ("inf", "inf")}, PINF32),
    ("minus_inf_times_inf", "fp16", 0, {7: ("-inf", "inf")}, NINF32),
    ("inf_beside_nan_product", "fp16", 0, {1: ("inf", "1"), 2: ("nan", "-1")}, NAN32),
    ("same_sign_infs", "fp16", PINF32, {4: ("inf", "1"), 12: ("-inf", "-1")}, PINF32),
    ("nan_times_zero", "fp16", 0, {0: ("nan", "0")}, NAN32),
    ("bf16_inf_times_zero", "bf16", 0, {8: (0x7F80, 0x0000)}, NAN32),
    ("bf16_inf_against_minus_inf_C", "bf16", NINF32, {0: (0x7F80, 0x4000)}, NAN32),
    ("bf16_minus_inf_product", "bf16", 0x3F800000, {0: (0xFF80, 0x4000)}, NINF32),
    ("e4m3_nan_times_zero", "e4m3", 0, {0: (0x7F, 0x00)}, NAN32),
    ("e4m3_negative_nan", "e4m3", 0, {0: (0xFF, 0x38)}, NAN32),
    ("e4m3_inf_C_absorbs_largest", "e4m3", PINF32, {k: (0x7E, 0x7E) for k in range(16)},
     PINF32),
    ("e4m3_minus_inf_C", "e4m3", NINF32, {0: (0x38, 0x38)}, NINF32),
]


def _special_dot(dtype, slots):
    cd = np.uint8 if dtype == "e4m3" else np.uint16
    a = np.zeros((1, 16), cd)
    b = np.zeros((1, 16), cd)
    for k, (x, y) in slots.items():
        a[0, k] = _F16[x] if isinstance(x, str) else x
        b[0, k] = _F16[y] if isinstance(y, str) else y
    return a, b


@pytest.mark.parametrize("case", SPECIAL_CASES, ids=[c[0] for c in SPECIAL_CASES])
def test_special_values_follow_ieee(orc, case):
    name, dtype, c, slots, want = case
    a, b = _special_dot(dtype, slots)
    for model in (["hopper"] if dtype == "e4m3" else ["ampere", "hopper"]):
        got = int(orc.dots(model, dtype, a, b, np.array([c], np.uint32))[0])
        assert got == want, f"{name} {model}: {got:#010x} != {want:#010x}"


@pytest.mark.parametrize("model", ["ampere", "hopper"])
def test_single_term_fp16_all_codes(orc, model):
    codes = np.arange(65536, dtype=np.uint16)
    got = _single_term(orc, model, "fp16", codes, 0x3C00)
    _assert_same_or_nan(got, codes.view(np.float16).astype(np.float32))


@pytest.mark.parametrize("model", ["ampere", "hopper"])
def test_single_term_bf16_all_codes(orc, model):
    codes = np.arange(65536, dtype=np.uint16)
    got = _single_term(orc, model, "bf16", codes, 0x3F80)
    _assert_same_or_nan(got, (codes.astype(np.uint32) << 16).view(np.float32))


def test_single_term_e4m3_all_codes(orc):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = _single_term(orc, "hopper", "e4m3", codes, 0x38)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    _assert_same_or_nan(got, ref)


def _two_term(orc, model, dtype, a0, b0):
    n = len(a0)
    cd = np.uint8 if dtype == "e4m3" else np.uint16
    nz = 0x80 if dtype == "e4m3" else 0x8000
    one = {"e4m3": 0x38, "fp16": 0x3C00, "bf16": 0x3F80}[dtype]
    a = np.full((n, 16), nz, cd)
    b = np.full((n, 16), one, cd)
    a[:, 5], b[:, 5] = a0, b0
    return orc.dots(model, dtype, a, b, np.full(n, 0x80000000, np.uint32))


def test_e4m3_all_products_exact(orc):
    """Every finite E4M3 product has at most 8 significant bits, so the
    emulated step must return it exactly (numpy float64 product)."""
    import torch
    fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    a0 = np.repeat(fin, fin.size)
    b0 = np.tile(fin, fin.size)
    vals = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn)
    vals = vals.to(torch.float64).numpy()
    ref = (vals[a0] * vals[b0]).astype(np.float32)
    got = _two_term(orc, "hopper", "e4m3", a0, b0)
    _assert_same_or_nan(got, ref)


@pytest.mark.parametrize("model", ["ampere", "hopper"])
def test_fp16_random_products_exact(orc, model):
    rng = np.random.default_rng(11)
    fin = np.nonzero((np.arange(65536) & 0x7C00) != 0x7C00)[0].astype(np.uint16)
    a0 = rng.choice(fin, 200000)
    b0 = rng.choice(fin, 200000)
    ref = (a0.view(np.float16).astype(np.float64) * b0.view(np.float16).astype(np.float64))
    got = _two_term(orc, model, "fp16", a0, b0)
    _assert_same_or_nan(got, ref.astype(np.float32))


@pytest.mark.parametrize("model", ["ampere", "hopper"])
def test_bf16_random_products_exact_or_inf(orc, model):
    rng = np.random.default_rng(12)
    fin = np.nonzero((np.arange(65536) & 0x7F80) != 0x7F80)[0].astype(np.uint16)
    a0 = rng.choice(fin, 200000)
    b0 = rng.choice(fin, 200000)
    va = (a0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vb = (b0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    p = va * vb
    got = _two_term(orc, model, "bf16", a0, b0)
    normal = (np.abs(p) >= 2.0 ** -126) & (np.abs(p) < 2.0 ** 128)
    assert normal.sum() > 50000
    _assert_same_or_nan(got[normal], p[normal].astype(np.float32))
    over = np.abs(p) >= 2.0 ** 128
    assert over.sum() > 1000
    want = np.where(p[over] > 0, 0x7F800000, 0xFF800000).astype(np.uint32)
    assert np.array_equal(got[over], want)


# ---------------------------------------- closed form: small integer GEMMs
@pytest.mark.parametrize("model,dtype", [("ampere", "fp16"), ("hopper", "fp16"),
                                         ("ampere", "bf16"), ("hopper", "bf16"),
                                         ("hopper", "e4m3")])
def test_integer_gemm_closed_form(orc, model, dtype):
    """With small integer inputs no bit is ever truncated (all terms are
    integers and every partial sum stays below 2^24 in magnitude), so the
    chained GEMM must equal C + A @ B computed in exact integer arithmetic.
    Catches dropped terms, wrong signs, transposed operands, wrong chaining."""
    import torch
    rng = np.random.default_rng(21)
    M, N, K = 19, 23, 80
    lim = 8 if dtype == "e4m3" else 64
    Ai = rng.integers(-lim, lim + 1, size=(M, K))
    Bi = rng.integers(-lim, lim + 1, size=(K, N))
    Ci = rng.integers(-(1 << 20), 1 << 20, size=(M, N))
    if dtype == "fp16":
        A = Ai.astype(np.float16).view(np.uint16)
        B = Bi.astype(np.float16).view(np.uint16)
    elif dtype == "bf16":
        A = (Ai.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        B = (Bi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    else:
        A = torch.from_numpy(Ai.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        B = torch.from_numpy(Bi.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    C = Ci.astype(np.float32).view(np.uint32)
    D, x = orc.gemm(model, dtype, A, B, C, nthreads=4)
    ref = (Ci + Ai @ Bi).astype(np.float32)
    # every prefix sum of the chain stays exact as well
    assert np.abs(Ci).max() + K * lim * lim < (1 << 24)
    assert np.array_equal(D.view(np.float32), ref)
    assert np.array_equal(x, np.bitwise_xor.reduce(D, axis=1))


# ------------------------------------------ oracle vs exact-rational model
def _random_dot_inputs(rng, dtype, n, adversarial):
    from bit_exact_matrix_amd import inputs as I
    if dtype == 2:
        a = I.e4m3_finite_codes(rng, (n, 16))
        b = I.e4m3_finite_codes(rng, (n, 16))
    elif adversarial:
        a = I._adversarial_elements(rng, dtype, (n, 16))
        b = I._adversarial_elements(rng, dtype, (n, 16))
    else:
        a = I.normal_codes(rng, dtype, (n, 16))
        b = I.normal_codes(rng, dtype, (n, 16))
    if adversarial:
        c = I._adversarial_c(rng, 0 if dtype == 2 else dtype, (n,))
    else:
        c = I.f32_bits(rng.standard_normal(n, dtype=np.float32))
    return a, b, c


@pytest.mark.parametrize("model,dtype", [(0, 0), (1, 0), (0, 1), (1, 1), (1, 2)])
@pytest.mark.parametrize("adversarial", [False, True])
def test_oracle_matches_rational_model(orc, model, dtype, adversarial):
    rng = np.random.default_rng(100 + 10 * model + dtype + (5 if adversarial else 0))
    n = 10000   # 10 cases: 100,000 single steps in all
    a, b, c = _random_dot_inputs(rng, dtype, n, adversarial)
    got = orc.dots(model, dtype, a, b, c)
    for r in range(n):
        want = RM.step(model, dtype, int(c[r]), [int(x) for x in a[r]], [int(x) for x in b[r]])
        assert int(got[r]) == want, (r, hex(int(got[r])), hex(want))


_SPECIALS = {0: (0x7C00, 0xFC00, 0x7C01, 0x0000, 0x8000),     # +inf -inf NaN +0 -0
             1: (0x7F80, 0xFF80, 0x7FC1, 0x0000, 0x8000),
             2: (None, None, 0x7F, 0x00, 0x80)}                 # E4M3: no infinities


@pytest.mark.parametrize("model,dtype", [(0, 0), (1, 0), (0, 1), (1, 1), (1, 2)])
def test_oracle_matches_rational_model_with_specials(orc, model, dtype):
    """inf, NaN and signed zeros (reading O12 and O11), oracle against the
    rational restatement: random steps with many special operands and C
    values, and steps whose inf/NaN products cancel exactly within one group
    ((-inf)*(-0) against (-0)*NaN, inf*x against NaN*(-x)): IEEE makes those
    NaN, however the fixed-width sums come out."""
    rng = np.random.default_rng(500 + 10 * model + dtype)
    n = 4000
    a, b, c = _random_dot_inputs(rng, dtype, n, True)
    pinf, ninf, nan, pz, nz = _SPECIALS[dtype]
    for x in (a, b):
        u = rng.random(x.shape)
        if pinf is not None:
            x[u < 0.02] = pinf
            x[(u >= 0.02) & (u < 0.04)] = ninf
        x[(u >= 0.04) & (u < 0.05)] = nan
        x[(u >= 0.05) & (u < 0.10)] = pz
        x[(u >= 0.10) & (u < 0.15)] = nz
    u = rng.random(n)
    c[u < 0.02] = 0x7F800000
    c[(u >= 0.02) & (u < 0.04)] = 0xFF800000
    c[(u >= 0.04) & (u < 0.05)] = 0x7FC00000
    c[(u >= 0.05) & (u < 0.10)] = 0x80000000
    # exact cancellations of inf/NaN products in the first group (k = 1, 2)
    big = ninf if ninf is not None else nan
    for r in range(0, 200):
        a[r, 1], b[r, 1], a[r, 2], b[r, 2] = big, nz, nz, nan
    for r in range(200, 400):
        a[r, 1], a[r, 2] = big, nan
        b[r, 2] = b[r, 1] ^ (0x80 if dtype == 2 else 0x8000)
    got = orc.dots(model, dtype, a, b, c)
    for r in range(n):
        want = RM.step(model, dtype, int(c[r]), [int(x) for x in a[r]], [int(x) for x in b[r]])
        assert int(got[r]) == want, (r, hex(int(got[r])), hex(want))
    assert np.all(got[:400] == 0x7FC00000)


@pytest.mark.parametrize("dtype", [0, 1])
def test_oracle_lovelace_matches_rational_ampere_model(orc, dtype):
    """The Lovelace model is the Ampere model ("Recovered Ampere FP16
    pipeline"): checked against the independent rational statement of it."""
    rng = np.random.default_rng(700 + dtype)
    n = 3000
    a, b, c = _random_dot_inputs(rng, dtype, n, True)
    got = orc.dots("lovelace", dtype, a, b, c)
    for r in range(n):
        want = RM.step(0, dtype, int(c[r]), [int(x) for x in a[r]], [int(x) for x in b[r]])
        assert int(got[r]) == want, (r, hex(int(got[r])), hex(want))


@pytest.mark.parametrize("model,dtype", [(0, 0), (1, 1), (1, 2)])
def test_oracle_gemm_chain_matches_rational_model(orc, model, dtype):
    from bit_exact_matrix_amd import inputs as I
    rng = np.random.default_rng(7 + model + dtype)
    if dtype == 2:
        A = I.e4m3_finite_codes(rng, (3, 48))
        B = I.e4m3_finite_codes(rng, (48, 3))
    else:
        A = I._adversarial_elements(rng, dtype, (3, 48))
        B = I._adversarial_elements(rng, dtype, (48, 3))
    C = I._adversarial_c(rng, 0 if dtype == 2 else dtype, (3, 3))
    D, _ = orc.gemm(model, dtype, A, B, C)
    assert np.array_equal(D, RM.gemm(model, dtype, A, B, C))


# ------------------------------------------------------------- invariants
def _codes_neg(x, dtype):
    return x ^ (np.uint8(0x80) if dtype == 2 else np.uint16(0x8000))


@pytest.mark.parametrize("model,dtype", [(0, 0), (1, 0), (0, 1), (1, 1), (1, 2)])
def test_sign_symmetry(orc, model, dtype):
    """D(-A, B, -C) is D(A, B, C) with the sign bit flipped (non-NaN, non-zero
    results); a two's-complement floor in place of magnitude truncation
    breaks it."""
    rng = np.random.default_rng(31 + model + dtype)
    a, b, c = _random_dot_inputs(rng, dtype, 40000, True)
    d1 = orc.dots(model, dtype, a, b, c)
    d2 = orc.dots(model, dtype, _codes_neg(a, dtype), b, c ^ np.uint32(0x80000000))
    ok = (d1 & 0x7FFFFFFF) != 0
    assert np.array_equal(d2[ok], d1[ok] ^ np.uint32(0x80000000))


@pytest.mark.parametrize("model,dtype", [(0, 0), (1, 0), (0, 1), (1, 1), (1, 2)])
def test_permutation_within_groups(orc, model, dtype):
    """Permuting products inside a group leaves D unchanged; moving a product
    across the Ampere stage boundary generally changes it."""
    rng = np.random.default_rng(41 + model + dtype)
    a, b, c = _random_dot_inputs(rng, dtype, 20000, False)
    d = orc.dots(model, dtype, a, b, c)
    groups = [list(range(8)), list(range(8, 16))] if model == 0 else [list(range(16))]
    perm = np.arange(16)
    for g in groups:
        perm[g] = rng.permutation(g)
    assert np.array_equal(orc.dots(model, dtype, a[:, perm], b[:, perm], c), d)
    if model == 0:
        swap = np.arange(16)
        swap[0], swap[8] = 8, 0
        assert not np.array_equal(orc.dots(model, dtype, a[:, swap], b[:, swap], c), d)


def test_power_of_two_scaling(orc):
    """Scaling A and C by 2^j (no subnormal or overflow involvement) scales D
    by exactly 2^j."""
    rng = np.random.default_rng(51)
    n = 20000
    from bit_exact_matrix_amd import inputs as I
    a = I.normal_codes(rng, 0, (n, 16))
    b = I.normal_codes(rng, 0, (n, 16))
    c = I.f32_bits(rng.standard_normal(n, dtype=np.float32))
    safe = ((a & 0x7C00) >= 0x0800).all(1) & ((a & 0x7C00) <= 0x6800).all(1) & \
           ((b & 0x7C00) != 0).all(1) & ((c & 0x7F800000) > 0x10000000)
    a, b, c = a[safe], b[safe], c[safe]
    for model in ("ampere", "hopper"):
        d = orc.dots(model, "fp16", a, b, c)
        for j in (-1, 3):
            a2 = (a.astype(np.int32) + (j << 10)).astype(np.uint16)
            c2 = (c.astype(np.int64) + (j << 23)).astype(np.uint32)
            d2 = orc.dots(model, "fp16", a2, b, c2)
            nz = (d & 0x7FFFFFFF) != 0
            assert np.array_equal(d2[nz], (d[nz].astype(np.int64) + (j << 23)).astype(np.uint32))


def test_tiles_and_xorsum(orc):
    """The tiles entry point equals 16x16 single-step GEMMs, and its xorsum is
    the XOR of the tile's 256 words."""
    from bit_exact_matrix_amd import inputs as I
    A, B, C = I.tiles_normal(1001, 7)
    D, x = orc.tiles("ampere", "fp16", A, B, C)
    for t in range(7):
        Dt, _ = orc.gemm("ampere", "fp16", A[t], B[t], C[t])
        assert np.array_equal(D[t], Dt)
    assert np.array_equal(x, np.bitwise_xor.reduce(D.reshape(7, 256), axis=1))
