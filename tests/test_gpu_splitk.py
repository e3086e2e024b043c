"""GPU split-K schedule (mma_emulate_gemm_splitk through the C ABI) against
the oracle's gemm_splitk, bit for bit: D and the xorsum of the final D."""
import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from bit_exact_matrix_amd import inputs as I
from test_gpu_parity import (COMBOS, DIGESTS, FULL, _gen, assert_bits_equal,  # noqa: F401
                             no_workspace, say, sha, to_dev, to_host_bits, torch_dev)

pytestmark = pytest.mark.gpu


def run_splitk(torch_dev, model, dt, A, B, C, splits, D=None):
    D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                   to_dev(torch_dev, C), D=D, xorsum=True, splits=splits)
    return to_host_bits(D), to_host_bits(X)


@pytest.mark.parametrize("model,dt", COMBOS)
@pytest.mark.parametrize("kind", ["normal", "specials"])
def test_splitk_matches_oracle(torch_dev, orc, model, dt, kind):
    for si, (M, N, K) in enumerate([(17, 33, 64), (130, 100, 256)]):
        A, B, C = _gen(kind, model, dt, M, N, K, 8000 + si)
        for splits in (1, 2, 4):
            say("split-K", model, dt, kind, (M, N, K), splits)
            got, gx = run_splitk(torch_dev, model, dt, A, B, C, splits)
            want, wx = orc.gemm_splitk(model, dt, A, B, C, splits)
            what = f"split-K {model}/{dt}/{kind} {M}x{N}x{K} splits={splits}"
            assert_bits_equal(got, want, what)
            assert_bits_equal(gx, wx, what + " xorsum")


def test_splitk_in_place_and_without_workspace(torch_dev, orc, no_workspace):
    torch, dev = torch_dev
    M, N, K = 70, 90, 128
    A, B, C = _gen("normal", "hopper", "bf16", M, N, K, 8100)
    want, wx = orc.gemm_splitk("hopper", "bf16", A, B, C, 8)
    tC = to_dev(torch_dev, C)
    say("split-K in place, no workspace")
    D, X = mm.gemm("hopper", "bf16", to_dev(torch_dev, A), to_dev(torch_dev, B), tC, D=tC,
                   xorsum=True, splits=8)
    assert_bits_equal(to_host_bits(D), want, "split-K in place")
    assert_bits_equal(to_host_bits(X), wx, "split-K in place xorsum")


def test_splitk_rejects_a_split_that_does_not_divide_the_steps(torch_dev):
    torch, dev = torch_dev
    A = torch.zeros((16, 48), dtype=torch.int16, device=dev)
    B = torch.zeros((48, 16), dtype=torch.int16, device=dev)
    for bad in (0, 2, 4):   # 48 / 16 = 3 steps
        with pytest.raises(mm.MmaEmuError):
            mm.gemm("ampere", "fp16", A, B, splits=bad)


def test_splitk_full_size(torch_dev, orc):
    """4096^3 FP16 Ampere with 4 runs of 64 steps: the whole output against
    the oracle's stored digest, and sampled rows recomputed here (rows are
    independent, so the oracle runs on those rows only)."""
    model, dt, gen = FULL["gemm_4096_fp16_ampere"]
    A, B, C = gen()
    say("split-K full size")
    got, gx = run_splitk(torch_dev, model, dt, A, B, C, 4)
    for r0, r1 in [(0, 2), (2047, 2049), (4094, 4096)]:
        want, wx = orc.gemm_splitk(model, dt, A[r0:r1], B, C[r0:r1], 4)
        assert_bits_equal(got[r0:r1], want, f"split-K full rows {r0}:{r1}")
        assert_bits_equal(gx[r0:r1], wx, f"split-K full xorsum rows {r0}:{r1}")
    d = DIGESTS["gemm_4096_fp16_ampere_splitk4"]
    assert sha(got) == d["D_sha256"], "split-K 4096^3: D differs from the oracle's"
    assert sha(gx) == d["xorsum_sha256"], "split-K 4096^3: xorsum differs from the oracle's"


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_many_runs_side_by_side(torch_dev, orc, model, dt):
    """Small M x N, long K: the runs are computed side by side into partial
    results and added in run order; up to one K-step per run.  In place too,
    and again with a workspace cap that forces the runs one after another."""
    import os
    torch, dev = torch_dev
    M, N, K = 70, 90, 1024                 # 64 K-steps
    A, B, C = _gen("specials", model, dt, M, N, K, 8200)
    for splits in (2, 16, 64):
        want, wx = orc.gemm_splitk(model, dt, A, B, C, splits)
        say("split-K side by side", model, dt, splits)
        got, gx = run_splitk(torch_dev, model, dt, A, B, C, splits)
        assert_bits_equal(got, want, f"side by side {model}/{dt} splits={splits}")
        assert_bits_equal(gx, wx, f"side by side {model}/{dt} splits={splits} xorsum")
        tC = to_dev(torch_dev, C)
        D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B), tC, D=tC,
                       xorsum=True, splits=splits)
        assert_bits_equal(to_host_bits(D), want, f"side by side in place splits={splits}")
        assert_bits_equal(to_host_bits(X), wx, f"side by side in place splits={splits} xorsum")
    # images of all 64 steps fit, the 16 partial results do not: runs in order
    os.environ["MMAEMU_WORKSPACE_MAX_BYTES"] = str(64 * 12 * 1024 * 4 + 4 * M * N * 4)
    try:
        want, wx = orc.gemm_splitk(model, dt, A, B, C, 16)
        got, gx = run_splitk(torch_dev, model, dt, A, B, C, 16)
    finally:
        del os.environ["MMAEMU_WORKSPACE_MAX_BYTES"]
    assert_bits_equal(got, want, f"runs in order {model}/{dt}")
    assert_bits_equal(gx, wx, f"runs in order {model}/{dt} xorsum")
