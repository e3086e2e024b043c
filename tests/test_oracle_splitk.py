"""Pins of the oracle's split-K schedule (oracle.gemm_splitk).

Hand-derived cases fix the reduction's rounding, order, zero sign and NaN;
the exact integer closed form must hold for every split count; one split is
the plain GEMM."""
import numpy as np
import pytest

from test_oracle_verify import _closed_form_case


def _one_output(K, entries, c_bits, dtype_code=np.uint16):
    A = np.zeros((1, K), dtype_code)
    B = np.zeros((K, 1), dtype_code)
    for k, (a, b) in entries.items():
        A[0, k], B[k, 0] = a, b
    return A, B, np.array([[c_bits]], np.uint32)


@pytest.mark.parametrize("model", ["ampere", "hopper"])
def test_second_run_rounds_to_nearest_even(orc, model):
    """C = 1 and, in the second K-step only, the product 1.5 * 2^-12 * 2^-11
    = 1.5 * 2^-23.  Chained, the step truncates it to one unit of 2^-23
    (Ampere: alignment onto the 2^-23 grid; Hopper: the round-toward-zero
    write-back): 1 + 2^-23 = 0x3F800001.  Split in two runs, the second run
    is exactly 1.5 * 2^-23 (0x34400000) and 1 + 1.5 ulp is a tie that goes
    to the even 1 + 2^-22 = 0x3F800002."""
    A, B, C = _one_output(32, {16: (0x0E00, 0x1000)}, 0x3F800000)
    D1, _ = orc.gemm(model, "fp16", A, B, C)
    D2, x2 = orc.gemm_splitk(model, "fp16", A, B, C, 2)
    assert int(D1[0, 0]) == 0x3F800001
    assert int(D2[0, 0]) == 0x3F800002
    assert int(x2[0]) == 0x3F800002
    # the second run alone, from +0
    P1, _ = orc.gemm(model, "fp16", A[:, 16:], B[16:, :], None)
    assert int(P1[0, 0]) == 0x34400000


def test_reduction_order_and_specials(orc):
    """Three runs: (P0 + P1) + P2 in that order.  P0 = 1, P1 = 2^-24,
    P2 = 2^-24: (1 + 2^-24) ties to 1, then again 1 -> 0x3F800000; the
    other association 1 + (2^-24 + 2^-24) would give 1 + 2^-23."""
    one_24 = (0x0C00, 0x0C00)           # 2^-12 * 2^-12 = 2^-24
    A, B, C = _one_output(48, {16: one_24, 32: one_24}, 0x3F800000)
    D, _ = orc.gemm_splitk("ampere", "fp16", A, B, C, 3)
    assert int(D[0, 0]) == 0x3F800000
    # +inf in run 0 and -inf in run 1: NaN, written canonically
    A, B, C = _one_output(32, {16: (0xFC00, 0x3C00)}, 0x7F800000)
    D, _ = orc.gemm_splitk("hopper", "fp16", A, B, C, 2)
    assert int(D[0, 0]) == 0x7FC00000
    # all terms -0: chained, every step is -0; split, run 1 starts from +0,
    # so it is +0 and -0 + +0 = +0
    A, B, C = _one_output(32, {k: (0x8000, 0x3C00) for k in range(32)}, 0x80000000)
    Dc, _ = orc.gemm("ampere", "fp16", A, B, C)
    Ds, _ = orc.gemm_splitk("ampere", "fp16", A, B, C, 2)
    assert int(Dc[0, 0]) == 0x80000000 and int(Ds[0, 0]) == 0x00000000


@pytest.mark.parametrize("model,dtype", [("ampere", "fp16"), ("hopper", "bf16"),
                                         ("hopper", "e4m3")])
def test_closed_form_holds_for_every_split(orc, model, dtype):
    rng = np.random.default_rng(88)
    A, B, C, exact = _closed_form_case(rng, dtype, 13, 29, 128)
    for splits in (1, 2, 4, 8):
        D, x = orc.gemm_splitk(model, dtype, A, B, C, splits)
        assert np.array_equal(D, exact), splits
        assert np.array_equal(x, np.bitwise_xor.reduce(exact, axis=1))


def test_one_split_is_the_plain_gemm(orc):
    from bit_exact_matrix_amd import inputs as I
    A, B, C = I.gemm_normal(3, 20, 30, 64, I.FP16, c_zero=False)
    D, x = orc.gemm("ampere", "fp16", A, B, C)
    D1, x1 = orc.gemm_splitk("ampere", "fp16", A, B, C, 1)
    assert np.array_equal(D, D1) and np.array_equal(x, x1)
