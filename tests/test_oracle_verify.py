"""Pins of the oracle's audit compare (oracle.verify / oracle.compare).

A claimed D that comes from outside the oracle -- the exact integer closed
form C + A @ B, valid when no bit is ever truncated -- must verify clean.
Planted differences must be reported exactly: their number, the smallest
planted index, and per row the XOR of the planted bit masks, all computed
here from the list of plants alone."""
import numpy as np
import pytest


def _closed_form_case(rng, dtype, M, N, K):
    import torch
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
    exact = (Ci + Ai @ Bi).astype(np.float32).view(np.uint32)
    return A, B, C, exact


def _plant(rng, D, n):
    """Flip random non-zero bit masks at n distinct random positions; return
    the claimed array and the plants {flat index: mask}."""
    claimed = D.copy().reshape(-1)
    idx = rng.choice(claimed.size, size=n, replace=False)
    masks = rng.integers(1, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    plants = {}
    for i, m in zip(idx.tolist(), masks.tolist()):
        claimed[i] ^= np.uint32(m)
        plants[i] = m
    return claimed.reshape(D.shape), plants


def _expected(plants, M, N):
    rows = [0] * M
    for i, m in plants.items():
        rows[i // N] ^= m
    return len(plants), (min(plants) if plants else None), np.array(rows, np.uint32)


@pytest.mark.parametrize("model,dtype", [("ampere", "fp16"), ("hopper", "bf16"),
                                         ("hopper", "e4m3")])
def test_verify_accepts_the_closed_form_and_reports_plants(orc, model, dtype):
    rng = np.random.default_rng(77)
    M, N, K = 21, 37, 64
    A, B, C, exact = _closed_form_case(rng, dtype, M, N, K)
    count, first, rows = orc.verify(model, dtype, A, B, C, exact, nthreads=4)
    assert (count, first) == (0, None)
    assert not rows.any()
    for n in (1, 2, 17, M * N):
        claimed, plants = _plant(rng, exact, n)
        count, first, rows = orc.verify(model, dtype, A, B, C, claimed, nthreads=4)
        ec, ef, er = _expected(plants, M, N)
        assert (count, first) == (ec, ef)
        assert np.array_equal(rows, er)


def test_compare_single_ulp_and_sign_of_zero():
    from oracle import compare
    D = np.array([[0x3F800000, 0x00000000], [0x7FC00000, 0xBF800000]], np.uint32)
    claimed = D.copy()
    claimed[0, 1] = 0x80000000          # -0 claimed for +0: a different bit pattern
    claimed[1, 1] = 0xBF800001          # one ulp away
    count, first, rows = compare(D, claimed)
    assert (count, first) == (2, 1)
    assert rows.tolist() == [0x80000000, 0x00000001]


def test_compare_empty():
    from oracle import compare
    D = np.zeros((3, 0), np.uint32)
    assert compare(D, D)[:2] == (0, None)
    assert compare(D, D)[2].tolist() == [0, 0, 0]


def test_row_words_have_the_xor_blind_spot_and_the_count_does_not():
    """One flipped bit changes exactly its row's word; the same flip in two
    elements of one row cancels in that row's word, while the mismatch
    count still sees both (the fingerprint's blind spot, documented)."""
    from oracle import compare
    D = (np.arange(12, dtype=np.uint32) + 0x3F800000).reshape(3, 4)
    claimed = D.copy()
    claimed[1, 0] ^= 0x10
    claimed[1, 3] ^= 0x10
    claimed[2, 2] ^= 0x4
    count, first, rows = compare(D, claimed)
    assert (count, first) == (3, 4)
    assert rows.tolist() == [0, 0, 0x4]
