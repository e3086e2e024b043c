"""mma_emulate_tiles at its edges, GPU against the oracle bit for bit:
batches that end in a partial group of tiles, C = NULL, C == D on
adversarial tiles (the exact recompute must read the original C), C, D
and the codes at addresses that are not 16-byte aligned (the scalar path),
and batches that follow a GEMM which left the LDS full of its own data."""
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


@pytest.mark.parametrize("model,dt", COMBOS)
def test_largest_group_sums(torch_dev, orc, model, dt):
    """Every significand all ones at one exponent, C a full FP32 significand
    at the products' exponent, all of one sign (then all negative, then
    alternating by tile): the largest sums a group forms (the bound that
    lets the kernel accumulate in 32 bits), in tiles and in a GEMM chain."""
    torch, dev = torch_dev
    one = {"fp16": 0x3FFF, "bf16": 0x3FFF, "e4m3": 0x3F}[dt]       # 1.11..1 x 2^0
    sign = {"fp16": 0x8000, "bf16": 0x8000, "e4m3": 0x80}[dt]
    code = np.uint8 if dt == "e4m3" else np.uint16
    n = 8
    A = np.full((n, 16, 16), one, code)
    B = np.full((n, 16, 16), one, code)
    C = np.full((n, 16, 16), 0x3FFFFFFF, np.uint32)                  # 1.11..1 x 2^0
    A[1::2] |= code(sign)                                             # negative products
    C[1::2] |= np.uint32(0x80000000)
    A[2:4] |= code(sign)
    B[2:4] |= code(sign)                                              # (-)(-): positive
    C[4:6] |= np.uint32(0x80000000)                                   # C against the products
    say("largest group sums", model, dt)
    D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                    to_dev(torch_dev, C), xorsum=True)
    _check(torch_dev, model, dt, A, B, C, D, X, orc, f"largest sums tiles {model}/{dt}")
    # the same operands as one 128 x 16 x 128 GEMM chain (eight steps)
    Ag = A.reshape(128, 16)
    Bg = np.ascontiguousarray(np.tile(B[0], (8, 8)))
    Cg = C.reshape(128, 16)[:, :16]
    Cg = np.ascontiguousarray(np.tile(Cg, (1, 8)))
    Ag = np.ascontiguousarray(np.tile(Ag, (1, 8)))
    want, wx = orc.gemm(model, dt, Ag, Bg, Cg)
    D, X = mm.gemm(model, dt, to_dev(torch_dev, Ag), to_dev(torch_dev, Bg),
                   to_dev(torch_dev, Cg), xorsum=True)
    assert_bits_equal(to_host_bits(D), want, f"largest sums gemm {model}/{dt}")
    assert_bits_equal(to_host_bits(X), wx, f"largest sums gemm xorsum {model}/{dt}")


def _cancelling_specials(model, dt, n_rows, seed):
    """A, B, C of shape n_rows x 64 x 32 (or tiles) in which every output of
    rows 0..3 has, in the first K-step, (-inf)*(-0) at k = 1 and (-0)*NaN at
    k = 2: two inf/NaN products with equal exponent codes and opposite
    signs, which cancel exactly in a fixed-width sum.  IEEE and the oracle
    make every such output NaN."""
    from test_gpu_parity import _gen
    A, B, C = _gen("normal", model, dt, n_rows, 64, 32, seed)
    if dt == "fp16":
        ninf, nzero, nan = 0xFC00, 0x8000, 0x7C01
    else:
        ninf, nzero, nan = 0xFF80, 0x8000, 0x7FC1
    A[0:4, 1], A[0:4, 2] = ninf, nzero
    B[1, :], B[2, :] = nzero, nan
    return A, B, C


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("ampere", "bf16"),
                                      ("hopper", "fp16")])
@pytest.mark.parametrize("variant", ["tiled", "tiled-no-workspace", "narrow", "narrow-lds",
                                     "spread2", "spread4"])
def test_cancelling_inf_nan_products(torch_dev, orc, model, dt, variant):
    import os
    A, B, C = _cancelling_specials(model, dt, 64, 9950)
    want, wx = orc.gemm(model, dt, A, B, C)
    assert np.all(want == 0x7FC00000), "the construction must give NaN everywhere"
    os.environ["MMAEMU_NARROW_BLOCKS"] = "0" if variant.startswith("tiled") else str(1 << 40)
    os.environ["MMAEMU_SPREAD_LANES"] = {"spread2": "2", "spread4": "4"}.get(variant, "0")
    if variant in ("tiled-no-workspace", "narrow-lds"):
        os.environ["MMAEMU_NO_WORKSPACE"] = "1"
    try:
        say("cancelling inf/NaN products", model, dt, variant)
        D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                       to_dev(torch_dev, C), xorsum=True)
        got, gx = to_host_bits(D), to_host_bits(X)
    finally:
        del os.environ["MMAEMU_NARROW_BLOCKS"]
        del os.environ["MMAEMU_SPREAD_LANES"]
        os.environ.pop("MMAEMU_NO_WORKSPACE", None)
    assert_bits_equal(got, want, f"cancelling specials {model}/{dt}/{variant}")
    assert_bits_equal(gx, wx, f"cancelling specials {model}/{dt}/{variant} xorsum")
    # the same first K-step as independent tiles
    At = np.ascontiguousarray(A[:64, :16].reshape(4, 16, 16))
    Bt = np.ascontiguousarray(np.broadcast_to(B[:16, :16], (4, 16, 16)))
    Ct = np.ascontiguousarray(C[:64, :16].reshape(4, 16, 16))
    wt, wtx = orc.tiles(model, dt, At, Bt, Ct)
    Dt, Xt = mm.tiles(model, dt, to_dev(torch_dev, At), to_dev(torch_dev, Bt),
                      to_dev(torch_dev, Ct), xorsum=True)
    assert_bits_equal(to_host_bits(Dt), wt, f"cancelling specials tiles {model}/{dt}")
    assert_bits_equal(to_host_bits(Xt), wtx, f"cancelling specials tiles {model}/{dt} xorsum")


@pytest.mark.parametrize("model,dt", COMBOS)
def test_tiles_after_a_gemm_left_lds_dirty(torch_dev, orc, model, dt):
    """Tile batches run right after a tiled GEMM on the same stream, whose
    operand images leave the LDS full of non-zero words: every LDS word the
    tile kernel reads must be one it wrote in this group of tiles (a stage
    word left partly unwritten would pick up the GEMM's data)."""
    import os
    os.environ["MMAEMU_NARROW_BLOCKS"] = "0"
    try:
        for n in (3, 66, 700):
            Ag, Bg, Cg = I.gemm_normal(9800 + n, 512, 512, 256, I.FP16, c_zero=False)
            mm.gemm("ampere", "fp16", to_dev(torch_dev, Ag), to_dev(torch_dev, Bg),
                    to_dev(torch_dev, Cg))
            A, B, C = _batch(9900 + n, n, dt)
            say("tiles after a GEMM", model, dt, n)
            D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                            to_dev(torch_dev, C), xorsum=True)
            _check(torch_dev, model, dt, A, B, C, D, X, orc, f"tiles after gemm {model}/{dt} n={n}")
    finally:
        del os.environ["MMAEMU_NARROW_BLOCKS"]
