"""GPU parity of the spread kernel (each output's products over 2 or 4
lanes, operand images from its own pre-pass) against the oracle, bit for
bit: chains whose length is not a whole number of the kernel's four LDS
stages, chains cut into chunks by a small workspace cap (each chunk
restarting from D), the audit compare under a cap too small for all of
its images (it then runs on the narrow kernel), and sampled rows of a
4096-step chain.  The GEMM parity, edge-case, ordered and verify suites
run on this kernel too (the gemm_kernel fixture)."""
import contextlib
import os

import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from bit_exact_matrix_amd import inputs as I
from test_gpu_parity import (COMBOS, _gen, assert_bits_equal, run_gemm, say, to_dev,  # noqa: F401
                             to_host_bits, torch_dev)

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def spread(lanes, cap=None):
    env = {"MMAEMU_NARROW_BLOCKS": str(1 << 40), "MMAEMU_SPREAD_LANES": str(lanes)}
    if cap is not None:
        env["MMAEMU_WORKSPACE_MAX_BYTES"] = str(cap)
    os.environ.update(env)
    try:
        yield
    finally:
        for k in env:
            del os.environ[k]


def step_bytes(lanes, M, N):
    """Workspace bytes of one chain position's images: 160 per row of A
    (rows padded to 16 / lanes) and per column of B (padded to 16)."""
    rows = -(-M // (16 // lanes)) * (16 // lanes)
    return (rows + -(-N // 16) * 16) * 160


@pytest.mark.parametrize("lanes", [2, 4])
@pytest.mark.parametrize("model,dt", COMBOS)
def test_spread_chain_lengths(torch_dev, orc, lanes, model, dt):
    """1 to 9 positions: no whole pass of four stages, one, two, and every
    remainder after them; ragged rows and columns."""
    for T in (1, 2, 3, 4, 5, 6, 7, 9):
        for kind in ("normal", "specials"):
            M, N, K = 5 + T, 37, 16 * T
            A, B, C = _gen(kind, model, dt, M, N, K, 15000 + T)
            say("spread", lanes, model, dt, kind, (M, N, K))
            with spread(lanes):
                got, gx = run_gemm(torch_dev, model, dt, A, B, C)
            want, wx = orc.gemm(model, dt, A, B, C)
            assert_bits_equal(got, want, f"spread{lanes} {model}/{dt}/{kind} {M}x{N}x{K}")
            assert_bits_equal(gx, wx, f"spread{lanes} xorsum {model}/{dt}/{kind} {M}x{N}x{K}")


@pytest.mark.parametrize("lanes", [2, 4])
def test_spread_in_chunks(torch_dev, orc, lanes):
    """A cap of three positions' images: the 10-position chain runs as
    chunks of 3, 3, 3 and 1, each from the D the one before wrote; in
    place too (D == C)."""
    M, N, K = 21, 50, 160
    for model, dt in COMBOS:
        A, B, C = _gen("wide", model, dt, M, N, K, 15100)
        want, wx = orc.gemm(model, dt, A, B, C)
        say("spread in chunks", lanes, model, dt)
        with spread(lanes, cap=3 * step_bytes(lanes, M, N)):
            got, gx = run_gemm(torch_dev, model, dt, A, B, C)
            tC = to_dev(torch_dev, C)
            D, _ = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B), tC, D=tC)
            inplace = to_host_bits(D)
        assert_bits_equal(got, want, f"spread{lanes} chunks {model}/{dt}")
        assert_bits_equal(gx, wx, f"spread{lanes} chunks xorsum {model}/{dt}")
        assert_bits_equal(inplace, want, f"spread{lanes} chunks in place {model}/{dt}")


@pytest.mark.parametrize("lanes", [2, 4])
def test_spread_audit_under_a_small_cap(torch_dev, orc, lanes):
    """The audit compare cannot restart from a D it does not store: under a
    cap that holds only some positions' images it takes the narrow kernel,
    with the same report."""
    M, N, K = 30, 40, 96
    A, B, C = _gen("normal", "hopper", "bf16", M, N, K, 15200)
    Dw, _ = orc.gemm("hopper", "bf16", A, B, C, xorsum=False)
    claimed = Dw.copy()
    claimed[7, 11] ^= np.uint32(1 << 3)
    claimed[29, 0] ^= np.uint32(1 << 30)
    want = orc.compare(Dw, claimed)
    for cap in (None, 2 * step_bytes(lanes, M, N)):
        say("spread audit", lanes, cap)
        with spread(lanes, cap=cap):
            report, X = mm.verify("hopper", "bf16", to_dev(torch_dev, A), to_dev(torch_dev, B),
                                  to_dev(torch_dev, C), to_dev(torch_dev, claimed),
                                  row_diff=True)
            got = mm.mismatches(report)
            gx = to_host_bits(X)
        assert got == want[:2], (got, want[:2], cap)
        assert_bits_equal(gx, want[2], f"spread{lanes} audit row xor, cap {cap}")


@pytest.mark.parametrize("lanes", [2, 4])
def test_spread_long_chain_sampled_rows(torch_dev, orc, lanes):
    """256 x 256 x 65536 (4096 chained K-steps), the shape the spread kernel
    is for: sampled rows against the oracle, and the fingerprint against
    the rows of D."""
    M, N, K = 256, 256, 65536
    A, B, C = I.gemm_normal(15300, M, N, K, I.FP16, c_zero=False)
    say("spread long chain", lanes)
    with spread(lanes):
        got, gx = run_gemm(torch_dev, "ampere", "fp16", A, B, C)
    assert np.array_equal(gx, np.bitwise_xor.reduce(got, axis=1))
    for r0, r1 in ((0, 2), (129, 130), (254, 256)):
        want, wx = orc.gemm_rows("ampere", "fp16", A, B, C, r0, r1)
        assert_bits_equal(got[r0:r1], want, f"spread{lanes} 256x256x65536 rows {r0}:{r1}")
        assert_bits_equal(gx[r0:r1], wx, f"spread{lanes} xorsum rows {r0}:{r1}")
