"""mma_emulate_tiles at its edges, GPU against the oracle bit for bit:
batches that end in a partial group of four tiles, C = NULL, C == D on
adversarial tiles (the exact recompute must read the original C), and C, D
and the codes at addresses that are not 16-byte aligned (the scalar path)."""
import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from bit_exact_matrix_amd import inputs as I
from test_gpu_parity import (COMBOS, DT, assert_bits_equal, say, to_dev,  # noqa: F401
                             to_host_bits, torch_dev)

pytestmark = pytest.mark.gpu


def _batch(seed, n, dt):
    """Half N(0,1), half adversarial (E4M3: every finite code, C adversarial)."""
    if dt != "e4m3":
        return I.tiles_mixed(seed, n, DT[dt])
    rng = I._rng(seed)
    A = I.e4m3_finite_codes(rng, (n, 16, 16))
    B = I.e4m3_finite_codes(rng, (n, 16, 16))
    return A, B, I._adversarial_c(rng, I.FP16, (n, 16, 16))


def _check(torch_dev, model, dt, A, B, C, D, X, orc, what):
    want, wx = orc.tiles(model, dt, A, B, C)
    assert_bits_equal(to_host_bits(D), want, what)
    assert_bits_equal(to_host_bits(X), wx, what + " xorsum")


@pytest.mark.parametrize("model,dt", COMBOS)
def test_partial_groups_and_null_c(torch_dev, orc, model, dt):
    for n in (1, 2, 3, 5, 7, 13, 66):
        A, B, C = _batch(9700 + n, n, dt)
        for c in (C, None):
            say("tiles", model, dt, n, "C=NULL" if c is None else "")
            D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                            to_dev(torch_dev, c), xorsum=True)
            _check(torch_dev, model, dt, A, B, c, D, X, orc, f"tiles {model}/{dt} n={n}")


@pytest.mark.parametrize("model,dt", COMBOS)
def test_in_place_on_adversarial_tiles(torch_dev, orc, model, dt):
    A, B, C = _batch(9800, 2002, dt)
    tC = to_dev(torch_dev, C)
    say("tiles in place", model, dt)
    D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B), tC, D=tC,
                    xorsum=True)
    assert D.data_ptr() == tC.data_ptr()
    _check(torch_dev, model, dt, A, B, C, D, X, orc, f"tiles in place {model}/{dt}")


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_unaligned_operands(torch_dev, orc, model, dt):
    """Every buffer one element past an aligned base."""
    torch, dev = torch_dev
    n = 1001
    A, B, C = _batch(9900, n, dt)

    def shifted(x, dtype):
        flat = torch.empty(x.size + 1, dtype=dtype, device=dev)
        flat[1:] = torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(
            {torch.int16: np.int16, torch.uint8: np.uint8, torch.float32: np.float32}[dtype])
        ).to(dev)
        return flat[1:].view(x.shape)

    code = torch.uint8 if dt == "e4m3" else torch.int16
    tA, tB, tC = shifted(A, code), shifted(B, code), shifted(C, torch.float32)
    tD = torch.empty(n * 256 + 1, dtype=torch.float32, device=dev)[1:].view(n, 16, 16)
    assert tC.data_ptr() % 16 and tD.data_ptr() % 16
    say("tiles unaligned", model, dt)
    D, X = mm.tiles(model, dt, tA, tB, tC, D=tD, xorsum=True)
    _check(torch_dev, model, dt, A, B, C, D, X, orc, f"tiles unaligned {model}/{dt}")
