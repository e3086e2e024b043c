"""Pins of two oracle entry points that the GPU comparisons lean on.

oracle.gemm_rows (mma_oracle_gemm_rows): a window of rows of the chained
GEMM.  Every large GPU comparison recomputes sampled rows with it, so it is
pinned on its own: on exact small-integer inputs each window must equal the
same rows of C + A @ B computed in integer arithmetic (a MatMul is a
deterministic sequence of tiles, Hawkeye notes "Key observations" 4, so a
row depends only on its own row of A and C), and on adversarial inputs it
must equal the rows of the full oracle GEMM, xorsum words included.

oracle.gemm_ordered: the K-steps of the chain taken in a given order (the
tile schedule the Hawkeye notes leave to later characterisation, "Critical
Analysis" and Future work 4).  Pinned by a hand-derived case in which the
reversed order keeps a truncated bit that the forward order loses, by the
exact closed form (which no order can change), and by the chain property."""
import numpy as np
import pytest

from bit_exact_matrix_amd import inputs as I
from test_oracle_verify import _closed_form_case

COMBOS = [("ampere", "fp16"), ("hopper", "fp16"), ("ampere", "bf16"), ("hopper", "bf16"),
          ("hopper", "e4m3")]
DT = {"fp16": I.FP16, "bf16": I.BF16, "e4m3": I.E4M3}


# ------------------------------------------------------------ gemm_rows
@pytest.mark.parametrize("model,dtype", COMBOS)
def test_row_windows_equal_the_exact_rows(orc, model, dtype):
    rng = np.random.default_rng(31)
    M, N, K = 23, 19, 96
    A, B, C, exact = _closed_form_case(rng, dtype, M, N, K)
    for (r0, r1), nth in (((3, 20), 3), ((0, 1), 1), ((M - 1, M), 4), ((0, M), 0),
                          ((5, 6), 8)):
        D, x = orc.gemm_rows(model, dtype, A, B, C, r0, r1, nthreads=nth)
        assert D.shape == (r1 - r0, N)
        assert np.array_equal(D, exact[r0:r1]), (r0, r1)
        assert np.array_equal(x, np.bitwise_xor.reduce(exact[r0:r1], axis=1)), (r0, r1)
    # an empty window is allowed and writes nothing
    D, x = orc.gemm_rows(model, dtype, A, B, C, 7, 7)
    assert D.shape == (0, N) and x.shape == (0,)


@pytest.mark.parametrize("model,dtype", COMBOS)
def test_row_windows_equal_the_full_gemm_on_adversarial_inputs(orc, model, dtype):
    for seed, mode in ((41, "wide"), (42, "coarse"), (43, "tiny")):
        A, B, C = I.gemm_adversarial(seed, 37, 29, 64, DT[dtype], mode)
        full, fx = orc.gemm(model, dtype, A, B, C, nthreads=4)
        for r0, r1 in ((0, 37), (3, 20), (0, 1), (36, 37), (17, 18)):
            D, x = orc.gemm_rows(model, dtype, A, B, C, r0, r1, nthreads=3)
            assert np.array_equal(D, full[r0:r1]), (mode, r0, r1)
            assert np.array_equal(x, fx[r0:r1]), (mode, r0, r1)
    A, B, C = I.gemm_specials(44, 21, 19, 48, DT[dtype])
    full, fx = orc.gemm(model, dtype, A, B, C)
    D, x = orc.gemm_rows(model, dtype, A, B, C, 4, 13, nthreads=2)
    assert np.array_equal(D, full[4:13]) and np.array_equal(x, fx[4:13])
    # C = NULL reads +0 for the window's rows as well
    full, fx = orc.gemm(model, dtype, A, B, None)
    D, x = orc.gemm_rows(model, dtype, A, B, None, 2, 9)
    assert np.array_equal(D, full[2:9]) and np.array_equal(x, fx[2:9])


def test_row_windows_outside_the_matrix_are_rejected(orc):
    A, B, C = I.gemm_normal(5, 8, 8, 32, I.FP16, c_zero=False)
    for r0, r1 in ((0, 9), (5, 4), (-1, 3)):
        with pytest.raises(ValueError):
            orc.gemm_rows("ampere", "fp16", A, B, C, r0, r1)


# ---------------------------------------------------------- gemm_ordered
def _three_steps(dtype):
    """One output, K = 48 (three steps), C = +0, one product per step:
    step 0 holds 1 * 1 = 1, steps 1 and 2 each 1.5 * 2^-12 * 2^-12 =
    1.5 * 2^-24 (FP16 0x3E00 * 0x3C00 scaled: 0x0E00 * 0x0C00; BF16 0x39C0 *
    0x3980), every other product +0."""
    one, a_small, b_small = ((0x3C00, 0x0E00, 0x0C00) if dtype == "fp16"
                             else (0x3F80, 0x39C0, 0x3980))
    A = np.zeros((1, 48), np.uint16)
    B = np.zeros((48, 1), np.uint16)
    A[0, 0], B[0, 0] = one, one
    for k in (16, 32):
        A[0, k], B[k, 0] = a_small, b_small
    return A, B


@pytest.mark.parametrize("model", ["ampere", "hopper"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_reversed_order_keeps_a_bit_the_forward_order_truncates(orc, model, dtype):
    """Forward (0, 1, 2): after step 0 the running value is 1.0; each small
    product is 0.75 units of the 2^-23 grid (Ampere's alignment) or 1.5
    units of 2^-24 (Hopper), which truncation at alignment or at the FP32
    write-back leaves below 2^-23: D = 1.0 = 0x3F800000.  Reversed (2, 1, 0):
    the two small products meet first and add exactly, 1.5 * 2^-23
    (0x34400000); against the product 1 it keeps one unit of 2^-23 after
    truncation: D = 1 + 2^-23 = 0x3F800001."""
    A, B = _three_steps(dtype)
    fwd, _ = orc.gemm_ordered(model, dtype, A, B, None, [0, 1, 2])
    rev, rx = orc.gemm_ordered(model, dtype, A, B, None, [2, 1, 0])
    assert int(fwd[0, 0]) == 0x3F800000
    assert int(rev[0, 0]) == 0x3F800001 and int(rx[0]) == 0x3F800001
    # the forward order is the plain chain
    plain, _ = orc.gemm(model, dtype, A, B, None)
    assert int(plain[0, 0]) == 0x3F800000
    # the first two positions of the reversed chain: exactly 1.5 * 2^-23
    two, _ = orc.gemm_ordered(model, dtype, A[:, 16:], B[16:, :], None, [1, 0])
    assert int(two[0, 0]) == 0x34400000


@pytest.mark.parametrize("model,dtype", COMBOS)
def test_no_order_changes_the_exact_closed_form(orc, model, dtype):
    rng = np.random.default_rng(97)
    A, B, C, exact = _closed_form_case(rng, dtype, 13, 17, 128)
    T = 8
    for order in (np.arange(T), np.arange(T)[::-1], rng.permutation(T), rng.permutation(T)):
        D, x = orc.gemm_ordered(model, dtype, A, B, C, order.astype(np.int32))
        assert np.array_equal(D, exact), order
        assert np.array_equal(x, np.bitwise_xor.reduce(exact, axis=1))


@pytest.mark.parametrize("model,dtype", COMBOS)
def test_an_ordered_chain_splits_into_two_chains(orc, model, dtype):
    """Chaining is sequential: the first h positions of an order, chained
    from C, then the rest chained from that result, give the whole chain
    (each part a plain gemm over the K-blocks it takes)."""
    rng = np.random.default_rng(5)
    A, B, C = I.gemm_adversarial(51, 21, 18, 160, DT[dtype], "narrow")
    order = rng.permutation(10).astype(np.int32)
    D, x = orc.gemm_ordered(model, dtype, A, B, C, order)

    def blocks(steps):
        cols = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in steps])
        return np.ascontiguousarray(A[:, cols]), np.ascontiguousarray(B[cols, :])

    for h in (1, 4, 9):
        A1, B1 = blocks(order[:h])
        D1, _ = orc.gemm(model, dtype, A1, B1, C)
        A2, B2 = blocks(order[h:])
        D2, x2 = orc.gemm(model, dtype, A2, B2, D1)
        assert np.array_equal(D2, D) and np.array_equal(x2, x), h
    # a different order changes this input's result
    other, _ = orc.gemm_ordered(model, dtype, A, B, C, np.arange(10, dtype=np.int32))
    assert not np.array_equal(other, D)
    # rows of an ordered chain
    Dr, xr = orc.gemm_ordered(model, dtype, A, B, C, order, rows=(3, 11))
    assert np.array_equal(Dr, D[3:11]) and np.array_equal(xr, x[3:11])


def test_order_entries_are_clamped_to_the_last_step(orc):
    """Reading: an entry read as an unsigned 32-bit integer at or past T
    (a negative int32 included) takes step T - 1."""
    A, B, C = I.gemm_normal(9, 6, 7, 48, I.FP16, c_zero=False)
    want, wx = orc.gemm_ordered("ampere", "fp16", A, B, C, np.array([0, 2, 2], np.int32))
    got, gx = orc.gemm_ordered("ampere", "fp16", A, B, C, np.array([0, 3, -1], np.int32))
    assert np.array_equal(got, want) and np.array_equal(gx, wx)
    with pytest.raises(AssertionError):
        orc.gemm_ordered("ampere", "fp16", A, B, C, np.array([0, 1], np.int32))
