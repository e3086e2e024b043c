"""Seeded adversarial GEMMs on random ragged shapes, GPU against the oracle
bit for bit: wide exponent ranges (overflow to inf states), narrow bands,
sums of signed powers of two that cancel to exact zeros mid-chain, and tiny
values whose results are FP32 subnormals or zero -- the cases the tiled
kernel hands to its exact per-output recompute."""
import zlib

import numpy as np
import pytest

import bit_exact_matrix_amd as mm  # noqa: F401
from bit_exact_matrix_amd import inputs as I
from test_gpu_parity import (COMBOS, DT, assert_bits_equal, gemm_kernel, no_workspace,  # noqa: F401
                             run_gemm, say, torch_dev)

pytestmark = pytest.mark.gpu

MODES = ["wide", "narrow", "coarse", "tiny"]


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 160)), int(rng.integers(1, 160)), 16 * int(rng.integers(1, 21)))
            for _ in range(n)]


@pytest.mark.parametrize("model,dt", COMBOS + [("lovelace", "bf16")])
@pytest.mark.parametrize("mode", MODES)
def test_adversarial_random_shapes(torch_dev, orc, gemm_kernel, model, dt, mode):
    for i, (M, N, K) in enumerate(_shapes(zlib.crc32(f"{model}/{dt}/{mode}".encode()), 6)):
        seed = 9000 + 100 * MODES.index(mode) + i
        A, B, C = I.gemm_adversarial(seed, M, N, K, DT[dt], mode)
        say("fuzz", model, dt, mode, (M, N, K), seed)
        got, gx = run_gemm(torch_dev, model, dt, A, B, C)
        want, wx = orc.gemm(model, dt, A, B, C)
        assert_bits_equal(got, want, f"fuzz {model}/{dt}/{mode} {M}x{N}x{K} seed {seed}")
        assert_bits_equal(gx, wx, f"fuzz xorsum {model}/{dt}/{mode} {M}x{N}x{K} seed {seed}")


@pytest.mark.parametrize("mode", MODES)
def test_adversarial_without_workspace(torch_dev, orc, no_workspace, mode):
    for i, (M, N, K) in enumerate(_shapes(777 + MODES.index(mode), 3)):
        for model, dt in (("ampere", "bf16"), ("hopper", "e4m3")):
            seed = 9500 + 10 * MODES.index(mode) + i
            A, B, C = I.gemm_adversarial(seed, M, N, K, DT[dt], mode)
            say("fuzz (no workspace)", model, dt, mode, (M, N, K), seed)
            got, gx = run_gemm(torch_dev, model, dt, A, B, C)
            want, wx = orc.gemm(model, dt, A, B, C)
            assert_bits_equal(got, want, f"fuzz/no-ws {model}/{dt}/{mode} {M}x{N}x{K}")
            assert_bits_equal(gx, wx, f"fuzz/no-ws xorsum {model}/{dt}/{mode} {M}x{N}x{K}")
