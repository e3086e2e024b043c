"""GPU audit compare (mma_verify_gemm through the C ABI) against the oracle.

The claimed D is the oracle's D (or, at 4096^3, the emulated D whose SHA-256
equals the oracle's stored digest) with planted bit flips.  The GPU's report
-- number of differing elements, smallest differing index, per-row XOR of
the differences -- must equal oracle.compare of the oracle's D with the
same claimed D, exactly."""
import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from test_gpu_parity import (COMBOS, DIGESTS, FULL, _gen, say, sha, to_dev,  # noqa: F401
                             to_host_bits, torch_dev, no_workspace, gemm_kernel)

pytestmark = pytest.mark.gpu


def _plant(rng, D, n):
    claimed = D.copy().reshape(-1)
    n = min(n, claimed.size)
    idx = rng.choice(claimed.size, size=n, replace=False)
    claimed[idx] ^= rng.integers(1, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    return claimed.reshape(D.shape)


def run_verify(torch_dev, model, dt, A, B, C, claimed, row_diff=True):
    report, X = mm.verify(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                          to_dev(torch_dev, C), to_dev(torch_dev, claimed), row_diff=row_diff)
    count, first = mm.mismatches(report)
    return count, first, (to_host_bits(X) if X is not None else None)


def check(torch_dev, orc, model, dt, A, B, C, D_oracle, claimed, what):
    want = orc.compare(D_oracle, claimed)
    got = run_verify(torch_dev, model, dt, A, B, C, claimed)
    assert got[:2] == want[:2], f"{what}: gpu {got[:2]} oracle {want[:2]}"
    assert np.array_equal(got[2], want[2]), f"{what}: row words differ"


@pytest.mark.parametrize("model,dt", COMBOS)
@pytest.mark.parametrize("kind", ["normal", "specials"])
def test_verify_matches_oracle(torch_dev, orc, gemm_kernel, model, dt, kind):
    rng = np.random.default_rng(4242)
    for si, (M, N, K) in enumerate([(17, 33, 48), (130, 100, 160), (129, 257, 96)]):
        A, B, C = _gen(kind, model, dt, M, N, K, 6000 + si)
        D, _ = orc.gemm(model, dt, A, B, C, xorsum=False)
        say("verify", model, dt, kind, (M, N, K))
        for n in (0, 1, 29, M * N):
            check(torch_dev, orc, model, dt, A, B, C, D, _plant(rng, D, n),
                  f"verify {model}/{dt}/{kind} {M}x{N}x{K} plants={n}")


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "bf16")])
def test_verify_in_place_unpack_path(torch_dev, orc, no_workspace, model, dt):
    rng = np.random.default_rng(99)
    M, N, K = 130, 100, 160
    A, B, C = _gen("normal", model, dt, M, N, K, 6100)
    D, _ = orc.gemm(model, dt, A, B, C, xorsum=False)
    say("verify (no workspace)", model, dt)
    for n in (0, 5):
        check(torch_dev, orc, model, dt, A, B, C, D, _plant(rng, D, n),
              f"verify/no-ws {model}/{dt} plants={n}")


def test_verify_k0_is_c_and_inputs_may_overlap(torch_dev, orc, gemm_kernel):
    """K = 0: the emulated D is C.  The claimed D may be the very buffer C."""
    torch, dev = torch_dev
    rng = np.random.default_rng(5)
    M, N = 40, 70
    A = np.zeros((M, 0), np.uint16)
    B = np.zeros((0, N), np.uint16)
    C = rng.integers(0, 1 << 32, size=(M, N), dtype=np.uint64).astype(np.uint32)
    say("verify K=0")
    check(torch_dev, orc, "ampere", "fp16", A, B, C, C, _plant(rng, C, 9), "verify K=0")
    tA, tB, tC = to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C)
    report, X = mm.verify("ampere", "fp16", tA, tB, tC, tC, row_diff=True)
    assert mm.mismatches(report) == (0, None)
    assert not to_host_bits(X).any()


def test_empty_rows_write_zero_words(torch_dev):
    """N = 0: nothing to compare or compute, but the M row words are written."""
    torch, dev = torch_dev
    M = 9
    A = torch.zeros((M, 16), dtype=torch.int16, device=dev)
    B = torch.zeros((16, 0), dtype=torch.int16, device=dev)
    say("empty rows")
    report, X = mm.verify("hopper", "fp16", A, B, None,
                          torch.zeros((M, 0), dtype=torch.float32, device=dev), row_diff=True)
    assert mm.mismatches(report) == (0, None)
    assert not to_host_bits(X).any()
    X = torch.full((M,), -1, dtype=torch.int32, device=dev)
    rc = mm.mma_emulate_gemm_async(1, 0, A.data_ptr(), B.data_ptr(), 0, 0, M, 0, 16,
                                   X.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert not to_host_bits(X).any()


@pytest.mark.parametrize("name", ["gemm_4096_fp16_ampere", "gemm_4096_e4m3_hopper"])
def test_verify_full_size(torch_dev, orc, name):
    """4096^3: the claimed D is the emulated D, which equals the oracle's
    (its digest is checked first), with planted flips whose report follows
    from oracle.compare against that same D."""
    torch, dev = torch_dev
    model, dt, gen = FULL[name]
    A, B, C = gen()
    say("verify full size", name)
    tA, tB, tC = to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C)
    tD, _ = mm.gemm(model, dt, tA, tB, tC)
    D = to_host_bits(tD)
    assert sha(D) == DIGESTS[name]["D_sha256"]
    rng = np.random.default_rng(11)
    for n in (0, 1000):
        claimed = _plant(rng, D, n)
        want = orc.compare(D, claimed)
        report, X = mm.verify(model, dt, tA, tB, tC, to_dev(torch_dev, claimed), row_diff=True)
        assert mm.mismatches(report) == want[:2]
        assert np.array_equal(to_host_bits(X), want[2])


def test_verify_xor_blind_spot(torch_dev, orc, gemm_kernel):
    """The same flip in two elements of one row: the row word cancels to 0,
    the count and first index still report both."""
    M, N, K = 20, 40, 32
    A, B, C = _gen("normal", "ampere", "fp16", M, N, K, 6200)
    D, _ = orc.gemm("ampere", "fp16", A, B, C, xorsum=False)
    claimed = D.copy()
    claimed[5, 3] ^= np.uint32(0x100)
    claimed[5, 30] ^= np.uint32(0x100)
    claimed[9, 0] ^= np.uint32(0x80000000)
    count, first, rows = run_verify(torch_dev, "ampere", "fp16", A, B, C, claimed)
    assert (count, first) == (3, 5 * N + 3)
    assert rows[5] == 0 and rows[9] == 0x80000000 and np.count_nonzero(rows) == 1
