"""Shapes at the library's limits, against the oracle on every output.

* M or N at the tiled kernel's grid limit (65,535 blocks of 64) and one block
  past it: a taller GEMM runs in row slices of that height, a wider one on
  the one-lane-per-output reference kernel, and so does split-K past the
  limit.  The rows of A and C (or the columns of B and C) repeat with
  period 61, so that D repeats with period 61 too and the oracle computes
  only one period; a row or column index that wraps at a power of two lands
  on a different residue mod 61 and shows.  At the limit the operand images
  exceed the workspace cap, so those calls also run in chunks of steps.
* A long chain: K = 65,536 (4096 chained steps) on one 64 x 64 block.
"""
import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from bit_exact_matrix_amd import inputs as I
from test_gpu_parity import (assert_bits_equal, gemm_kernel, say, to_dev,  # noqa: F401
                             to_host_bits, torch_dev)

pytestmark = pytest.mark.gpu

PERIOD = 61
LIMIT = 65535 * 64          # rows (or columns) of the largest tiled grid


def _periodic(a, reps, axis):
    shape = [1, 1]
    shape[axis] = reps
    return np.tile(a, shape)


@pytest.mark.parametrize("rows", [LIMIT, LIMIT + 64, LIMIT + 1000])
def test_tall_gemm_at_the_grid_limit(torch_dev, orc, rows):
    N, K = 16, 32
    A0, B, C0 = I.gemm_normal(9300, PERIOD, N, K, I.FP16, c_zero=False)
    reps = -(-rows // PERIOD)
    A = _periodic(A0, reps, 0)[:rows]
    C = _periodic(C0, reps, 0)[:rows]
    D0, x0 = orc.gemm("ampere", "fp16", A0, B, C0)
    say("tall gemm", rows, N, K)
    D, X = mm.gemm("ampere", "fp16", to_dev(torch_dev, A), to_dev(torch_dev, B),
                   to_dev(torch_dev, C), xorsum=True)
    assert_bits_equal(to_host_bits(D), _periodic(D0, reps, 0)[:rows], f"tall {rows} rows")
    assert_bits_equal(to_host_bits(X), np.tile(x0, reps)[:rows], f"tall {rows} rows xorsum")


@pytest.mark.parametrize("cols", [LIMIT, LIMIT + 64])
def test_wide_gemm_at_the_grid_limit(torch_dev, orc, cols):
    M, K = 16, 32
    A, B0, C0 = I.gemm_normal(9400, M, PERIOD, K, I.BF16, c_zero=False)
    reps = -(-cols // PERIOD)
    B = _periodic(B0, reps, 1)[:, :cols]
    C = _periodic(C0, reps, 1)[:, :cols]
    D0, _ = orc.gemm("hopper", "bf16", A, B0, C0)
    want = _periodic(D0, reps, 1)[:, :cols]
    say("wide gemm", M, cols, K)
    D, X = mm.gemm("hopper", "bf16", to_dev(torch_dev, A), to_dev(torch_dev, B),
                   to_dev(torch_dev, C), xorsum=True)
    assert_bits_equal(to_host_bits(D), want, f"wide {cols} columns")
    # the row words over the full width, by their definition
    assert_bits_equal(to_host_bits(X), np.bitwise_xor.reduce(want, axis=1),
                      f"wide {cols} columns xorsum")


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "e4m3")])
def test_long_chain(torch_dev, orc, gemm_kernel, model, dt):
    M, N, K = 64, 64, 65536
    A, B, C = (I.gemm_e4m3(9500, M, N, K) if dt == "e4m3"
               else I.gemm_normal(9500, M, N, K, I.FP16, c_zero=False))
    want, wx = orc.gemm(model, dt, A, B, C)
    say("long chain", model, dt, K)
    D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                   to_dev(torch_dev, C), xorsum=True)
    assert_bits_equal(to_host_bits(D), want, f"long chain {model}/{dt}")
    assert_bits_equal(to_host_bits(X), wx, f"long chain {model}/{dt} xorsum")


def test_split_k_past_the_grid_limit(torch_dev, orc):
    """Split-K on a shape the tiled kernel does not take: the one-lane-per-
    output kernel runs the two runs in order and adds the second into D."""
    rows, N, K = LIMIT + 64, 16, 32
    A0, B, C0 = I.gemm_normal(9450, PERIOD, N, K, I.FP16, c_zero=False)
    reps = -(-rows // PERIOD)
    A = _periodic(A0, reps, 0)[:rows]
    C = _periodic(C0, reps, 0)[:rows]
    D0, x0 = orc.gemm_splitk("hopper", "fp16", A0, B, C0, 2)
    say("split-K past the grid limit", rows, N, K)
    D, X = mm.gemm("hopper", "fp16", to_dev(torch_dev, A), to_dev(torch_dev, B),
                   to_dev(torch_dev, C), xorsum=True, splits=2)
    assert_bits_equal(to_host_bits(D), _periodic(D0, reps, 0)[:rows], "split-K tall")
    assert_bits_equal(to_host_bits(X), np.tile(x0, reps)[:rows], "split-K tall xorsum")
