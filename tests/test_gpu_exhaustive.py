"""Every operand code through the GPU kernels, against the oracle.

Row i of A holds code i of the format in slot k = i mod 16, so that every
FP16 and BF16 code (subnormals, signed zeros, infinities and every NaN
payload included) is taken in each of the 16 product slots, both Ampere
stages alike.  "Isolated": the other slots and C hold +0 codes, and every B
column carries one of the codes below, so D = one product, and each A code
meets each of those B codes (for E4M3, all 256 codes: every product of two
codes).  "Isolated-b" is its mirror image, with every code in B.
"Embedded": A's other slots, all of B and C are random finite values, so
each A code's product is summed with 15 others and C.  Each case runs
through all three operand decoders and is compared with the oracle bit for
bit.  Two more tests sweep C (every FP32 exponent field, with 128
fractions and both signs) and take every code through the tile batches.
"""
import numpy as np
import pytest

import os

from test_gpu_parity import assert_bits_equal, run_gemm, say, torch_dev  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["tiled", "tiled-in-lds", "narrow", "narrow-lds", "spread"])
def kernel(request):
    """The operand decoders: the tiled kernel's pre-pass (operand images in
    a workspace), its in-LDS image builder (no workspace; the tile batches
    use the same builder), the narrow kernel's own (B always; A without a
    workspace) and the spread kernel's pre-pass (one image per row or
    column; also the narrow kernel's A when there is a workspace)."""
    env = {"tiled": {"MMAEMU_NARROW_BLOCKS": "0"},
           "tiled-in-lds": {"MMAEMU_NARROW_BLOCKS": "0", "MMAEMU_NO_WORKSPACE": "1"},
           "narrow": {"MMAEMU_NARROW_BLOCKS": str(1 << 40), "MMAEMU_SPREAD_LANES": "0"},
           "narrow-lds": {"MMAEMU_NARROW_BLOCKS": str(1 << 40), "MMAEMU_SPREAD_LANES": "0",
                          "MMAEMU_NO_WORKSPACE": "1"},
           "spread": {"MMAEMU_NARROW_BLOCKS": str(1 << 40),
                      "MMAEMU_SPREAD_LANES": "2"}}[request.param]
    os.environ.update(env)
    yield request.param
    for k in env:
        del os.environ[k]

# B codes met by every A code: one, minus one, the largest finite value, the
# smallest and largest subnormal, the smallest normal, +0, -0, +inf, -inf,
# a quiet NaN, a value just below two, and a negative mid-range value
B_CODES = {
    "fp16": [0x3C00, 0xBC00, 0x7BFF, 0x0001, 0x03FF, 0x0400, 0x0000, 0x8000, 0x7C00, 0xFC00,
             0x7E00, 0x3FFF, 0xC555],
    "bf16": [0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x007F, 0x0080, 0x0000, 0x8000, 0x7F80, 0xFF80,
             0x7FC0, 0x3FFF, 0xC2AA],
}
N_RANDOM = 27          # further random B codes: 40 in all (ragged tile edges)


def _finite_codes(rng, dt, shape):
    if dt == "fp16":
        return rng.standard_normal(shape).astype(np.float16).view(np.uint16)
    if dt == "bf16":
        f = rng.standard_normal(shape).astype(np.float32).view(np.uint32)
        return (f >> 16).astype(np.uint16)
    c = rng.integers(0, 256, shape, dtype=np.uint16)
    c[(c & 0x7F) == 0x7F] = 0x38          # E4M3's only NaN codes -> 1.0
    return c.astype(np.uint8)


def _inputs(dt, mode, seed):
    """A, B and C (None for +0) of one case; row i of A holds code i of the
    format (all 256 for E4M3) in slot i mod 16."""
    rng = np.random.default_rng(seed)
    K = 16
    cd = np.uint8 if dt == "e4m3" else np.uint16
    M = 256 if dt == "e4m3" else 65536
    a_codes = np.arange(M, dtype=np.uint32).astype(cd)
    if dt == "e4m3":
        b_row = np.arange(256, dtype=np.uint32).astype(cd)
    else:
        extra = rng.integers(0, 65536, N_RANDOM, dtype=np.uint32).astype(cd)
        b_row = np.concatenate([np.array(B_CODES[dt], cd), extra])
    nb = len(b_row)
    if mode in ("isolated", "isolated-b"):
        # column block k carries the B codes in slot k and +0 elsewhere: in
        # block (i mod 16) row i's product with each B code is the only term
        # that is not 0 * 0
        A = np.zeros((M, K), cd)
        B = np.zeros((K, K * nb), cd)
        for k in range(K):
            B[k, k * nb:(k + 1) * nb] = b_row
        C = None
    else:
        A = _finite_codes(rng, dt, (M, K)).astype(cd)
        B = _finite_codes(rng, dt, (K, nb)).astype(cd)
        C = rng.standard_normal((M, nb)).astype(np.float32).view(np.uint32)
    A[np.arange(M), np.arange(M) % K] = a_codes
    if mode == "isolated-b":
        # the mirror image: column j of B holds code j in slot j mod 16, and
        # row block k of A the codes above in slot k
        A, B = np.ascontiguousarray(B.T), np.ascontiguousarray(A.T)
    return A, B, C


@pytest.mark.parametrize("mode", ["isolated", "isolated-b", "embedded"])
@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "fp16"),
                                      ("ampere", "bf16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_every_operand_code(torch_dev, orc, kernel, model, dt, mode):
    A, B, C = _inputs(dt, mode, 9700 + 10 * ("fp16", "bf16", "e4m3").index(dt)
                      + ("isolated", "isolated-b", "embedded").index(mode))
    say("every operand code", model, dt, mode, kernel, A.shape, B.shape)
    want, wx = orc.gemm(model, dt, A, B, C)
    got, gx = run_gemm(torch_dev, model, dt, A, B, C)
    what = f"every {dt} code, {model}, {mode}, {kernel} kernel"
    assert_bits_equal(got, want, what)
    assert_bits_equal(gx, wx, what + " xorsum")


def _c_words(rng):
    """65,536 FP32 words: every exponent field (0 for zeros and subnormals,
    255 for infinities and NaNs) with 128 fractions each (0, 1, the largest,
    the top bit alone, and random ones), both signs."""
    fr = np.concatenate([np.array([0, 1, 0x7FFFFF, 0x400000], np.uint32),
                         rng.integers(0, 1 << 23, 124, dtype=np.uint32)])
    e = np.arange(256, dtype=np.uint32)
    s = np.array([0, 1], np.uint32)
    w = (s[:, None, None] << 31) | (e[None, :, None] << 23) | fr[None, None, :]
    return w.reshape(1024, 64)


@pytest.mark.parametrize("mode", ["alone", "summed"])
@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_every_c_exponent(torch_dev, orc, kernel, model, dt, mode):
    """C through the state decode and encode: alone (every product 0 * 0),
    or summed with 16 random finite products."""
    rng = np.random.default_rng(9800 + ("alone", "summed").index(mode))
    C = _c_words(rng)
    M, N, K = C.shape[0], C.shape[1], 16
    cd = np.uint8 if dt == "e4m3" else np.uint16
    if mode == "alone":
        A, B = np.zeros((M, K), cd), np.zeros((K, N), cd)
    else:
        A, B = (_finite_codes(rng, dt, (M, K)).astype(cd),
                _finite_codes(rng, dt, (K, N)).astype(cd))
    say("every C exponent", model, dt, mode, kernel)
    want, wx = orc.gemm(model, dt, A, B, C)
    got, gx = run_gemm(torch_dev, model, dt, A, B, C)
    what = f"every C exponent, {model}/{dt}, {mode}, {kernel} kernel"
    assert_bits_equal(got, want, what)
    assert_bits_equal(gx, wx, what + " xorsum")


@pytest.mark.parametrize("side", ["a", "b"])
@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "fp16"),
                                      ("ampere", "bf16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_every_operand_code_in_tiles(torch_dev, orc, model, dt, side):
    """The tile batches: code i of the format sits in tile i // 16 (for E4M3
    the 256 codes repeat over 16 tiles), row (A) or column (B) i mod 16, at
    slot (i + i // 16) mod 16; the rest of A and B and all of C are random
    finite values."""
    import bit_exact_matrix_amd as mm
    from test_gpu_parity import to_dev, to_host_bits
    rng = np.random.default_rng(9900 + 2 * ("fp16", "bf16", "e4m3").index(dt) + (side == "b"))
    cd = np.uint8 if dt == "e4m3" else np.uint16
    n = 4096 if dt != "e4m3" else 256
    codes = np.arange(16 * n, dtype=np.uint32).astype(cd)
    A = _finite_codes(rng, dt, (n, 16, 16)).astype(cd)
    B = _finite_codes(rng, dt, (n, 16, 16)).astype(cd)
    C = rng.standard_normal((n, 16, 16)).astype(np.float32).view(np.uint32)
    i = np.arange(16 * n)
    t, r, k = i // 16, i % 16, (i + i // 16) % 16
    if side == "a":
        A[t, r, k] = codes
    else:
        B[t, k, r] = codes
    say("every operand code in tiles", model, dt, side)
    want, wx = orc.tiles(model, dt, A, B, C)
    D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                    to_dev(torch_dev, C), xorsum=True)
    what = f"every {dt} code in tiles, {model}, side {side}"
    assert_bits_equal(to_host_bits(D), want, what)
    assert_bits_equal(to_host_bits(X), wx, what + " xorsum")
