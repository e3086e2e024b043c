"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle,
bit for bit, on the same seeded inputs.

Small and medium cases compare every output with the oracle computed here.
The full-size workloads (4096^3 GEMMs, 100,000-tile batches) compare the
SHA-256 of every output word with digests the oracle wrote
(tests/golden/oracle_digests.json, made by tests/golden/make_digests.py),
and in addition recompute sampled rows with the oracle on the spot.
"""
import hashlib
import json
import os

import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from bit_exact_matrix_amd import inputs as I

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DIGESTS_PATH = os.path.join(HERE, "golden", "oracle_digests.json")
DIGESTS = json.load(open(DIGESTS_PATH)) if os.path.exists(DIGESTS_PATH) else {}
COMBOS = [("ampere", "fp16"), ("hopper", "fp16"), ("ampere", "bf16"), ("hopper", "bf16"),
          ("hopper", "e4m3")]
DT = {"fp16": I.FP16, "bf16": I.BF16, "e4m3": I.E4M3}


def say(*a):
    print("[gpu-parity]", *a, flush=True)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.load_library()
    return torch, torch.device("cuda:0")


def to_dev(torch_dev, x):
    torch, dev = torch_dev
    if x is None:
        return None
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    elif x.dtype == np.uint32:
        x = x.view(np.float32)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def to_host_bits(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint32)


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def run_gemm(torch_dev, model, dt, A, B, C, xorsum=True):
    D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                   to_dev(torch_dev, C), xorsum=xorsum)
    return to_host_bits(D), (to_host_bits(X) if X is not None else None)


def assert_bits_equal(got, want, what):
    if not np.array_equal(got, want):
        idx = np.argwhere(got != want)
        first = tuple(idx[0])
        raise AssertionError(f"{what}: {len(idx)} of {got.size} words differ; first at {first}: "
                             f"gpu {int(got[first]):#010x} oracle {int(want[first]):#010x}")


# --------------------------------------------------------------- tiles
def test_tiles_1k_fp16_ampere(torch_dev, orc):
    A, B, C = I.tiles_normal(1001, 1000)
    say("tiles 1k fp16 ampere")
    want, wx = orc.tiles("ampere", "fp16", A, B, C)
    D, X = mm.tiles("ampere", "fp16", to_dev(torch_dev, A), to_dev(torch_dev, B),
                    to_dev(torch_dev, C), xorsum=True)
    assert_bits_equal(to_host_bits(D), want, "tiles D")
    assert_bits_equal(to_host_bits(X), wx, "tiles xorsum")
    d = DIGESTS.get("tiles_fp16_1k_ampere")
    if d:
        assert sha(want) == d["D_sha256"] and sha(wx) == d["xorsum_sha256"]


@pytest.mark.parametrize("model,dt", COMBOS[:4])
def test_tiles_mixed_100k(torch_dev, orc, model, dt):
    """100,000 tiles, half N(0,1), half adversarial, all D words compared."""
    seed = 2001 if dt == "fp16" else 2002
    A, B, C = I.tiles_mixed(seed, 100000, DT[dt])
    say("tiles mixed 100k", model, dt)
    D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                    to_dev(torch_dev, C), xorsum=True)
    got, gx = to_host_bits(D), to_host_bits(X)
    want, wx = orc.tiles(model, dt, A, B, C)
    assert_bits_equal(got, want, f"tiles {model}/{dt}")
    assert_bits_equal(gx, wx, f"tiles xorsum {model}/{dt}")
    d = DIGESTS.get(f"tiles_mixed_100k_{dt}_{model}")
    if d:
        assert sha(got) == d["D_sha256"] and sha(gx) == d["xorsum_sha256"]


def test_tiles_specials_and_null_c(torch_dev, orc):
    for model, dt in COMBOS:
        A, B, C = I.gemm_specials(61, 16 * 40, 16, 16, DT[dt])
        A = A.reshape(40, 16, 16)
        B = np.ascontiguousarray(np.broadcast_to(B, (40, 16, 16)))
        C = C.reshape(40, 16, 16)
        for c in (C, None):
            say("tiles specials", model, dt, "C" if c is not None else "C=NULL")
            want, wx = orc.tiles(model, dt, A, B, c)
            D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                            to_dev(torch_dev, c), xorsum=True)
            assert_bits_equal(to_host_bits(D), want, f"tiles specials {model}/{dt}")
            assert_bits_equal(to_host_bits(X), wx, f"tiles specials xorsum {model}/{dt}")


# -------------------------------------------------- GEMM, oracle-sized
SHAPES = [(1, 1, 16), (16, 16, 16), (17, 33, 48), (64, 64, 64), (130, 100, 160),
          (257, 65, 32), (129, 257, 96)]


def _gen(kind, model, dt, M, N, K, seed):
    if kind == "normal":
        if dt == "e4m3":
            return I.gemm_e4m3(seed, M, N, K)
        return I.gemm_normal(seed, M, N, K, DT[dt], c_zero=False)
    if kind == "wide":
        if dt == "bf16":
            return I.gemm_wide_bf16(seed, M, N, K)
        return _gen("normal", model, dt, M, N, K, seed)
    return I.gemm_specials(seed, M, N, K, DT[dt])


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_lovelace_gemm_and_tiles(torch_dev, orc, gemm_kernel, dt):
    """Lovelace runs the Ampere arithmetic: GEMMs and tiles against the
    oracle's Lovelace model."""
    for si, (M, N, K) in enumerate([(17, 33, 48), (130, 100, 160)]):
        for kind in ("normal", "specials"):
            A, B, C = _gen(kind, "lovelace", dt, M, N, K, 7000 + si)
            say("lovelace gemm", dt, kind, (M, N, K))
            got, gx = run_gemm(torch_dev, "lovelace", dt, A, B, C)
            want, wx = orc.gemm("lovelace", dt, A, B, C)
            assert_bits_equal(got, want, f"lovelace {dt}/{kind} {M}x{N}x{K}")
            assert_bits_equal(gx, wx, f"lovelace xorsum {dt}/{kind} {M}x{N}x{K}")
    A, B, C = I.tiles_normal(1001, 300) if dt == "fp16" else I.tiles_mixed(2002, 300, I.BF16)
    D, X = mm.tiles("lovelace", dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                    to_dev(torch_dev, C), xorsum=True)
    want, wx = orc.tiles("lovelace", dt, A, B, C)
    assert_bits_equal(to_host_bits(D), want, f"lovelace tiles {dt}")
    assert_bits_equal(to_host_bits(X), wx, f"lovelace tiles xorsum {dt}")


@pytest.mark.parametrize("model,dt", COMBOS)
@pytest.mark.parametrize("kind", ["normal", "wide", "specials"])
def test_gemm_small_full_compare(torch_dev, orc, gemm_kernel, model, dt, kind):
    for si, (M, N, K) in enumerate(SHAPES):
        A, B, C = _gen(kind, model, dt, M, N, K, 1000 + si)
        say("gemm", model, dt, kind, (M, N, K))
        got, gx = run_gemm(torch_dev, model, dt, A, B, C)
        want, wx = orc.gemm(model, dt, A, B, C)
        assert_bits_equal(got, want, f"gemm {model}/{dt}/{kind} {M}x{N}x{K}")
        assert_bits_equal(gx, wx, f"gemm xorsum {model}/{dt}/{kind} {M}x{N}x{K}")


@pytest.mark.parametrize("model,dt", COMBOS)
def test_gemm_edge_cases(torch_dev, orc, gemm_kernel, model, dt):
    torch, dev = torch_dev
    M, N, K = 33, 47, 64
    A, B, C = _gen("normal", model, dt, M, N, K, 77)
    # C = NULL means +0
    say("edge C=NULL", model, dt)
    D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B), None, xorsum=True)
    want, wx = orc.gemm(model, dt, A, B, None)
    assert_bits_equal(to_host_bits(D), want, "C=NULL")
    assert_bits_equal(to_host_bits(X), wx, "C=NULL xorsum")
    # in place: D == C
    say("edge in-place", model, dt)
    tC = to_dev(torch_dev, C)
    D, _ = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B), tC, D=tC)
    want, _ = orc.gemm(model, dt, A, B, C)
    assert D.data_ptr() == tC.data_ptr()
    assert_bits_equal(to_host_bits(D), want, "in-place")
    # K = 0: D = C, xorsum of C
    say("edge K=0", model, dt)
    cd = 1 if dt == "e4m3" else 2
    z = np.zeros((M, 0), np.uint8 if cd == 1 else np.uint16)
    zb = np.zeros((0, N), np.uint8 if cd == 1 else np.uint16)
    tA = torch.empty((M, 0), dtype=torch.uint8 if cd == 1 else torch.int16, device=dev)
    tB = torch.empty((0, N), dtype=torch.uint8 if cd == 1 else torch.int16, device=dev)
    D, X = mm.gemm(model, dt, tA, tB, to_dev(torch_dev, C), xorsum=True)
    assert_bits_equal(to_host_bits(D), C, "K=0")
    want, wx = orc.gemm(model, dt, z, zb, C)
    assert_bits_equal(to_host_bits(X), wx, "K=0 xorsum")
    # M = 0 and N = 0 do nothing
    D, X = mm.gemm(model, dt, tA[:0], tB, None, xorsum=True)
    assert D.shape == (0, N)


# ------------------------------------------------ full-size workloads
FULL = {
    "gemm_4096_fp16_ampere": ("ampere", "fp16", lambda: I.gemm_normal(3001, 4096, 4096, 4096)),
    "gemm_4096_bf16_hopper": ("hopper", "bf16", lambda: I.gemm_wide_bf16(4001, 4096, 4096, 4096)),
    "gemm_4096_e4m3_hopper": ("hopper", "e4m3", lambda: I.gemm_e4m3(5001, 4096, 4096, 4096)),
}
SAMPLE_ROWS = [(0, 2), (15, 18), (1000, 1001), (2047, 2049), (4094, 4096)]


@pytest.mark.parametrize("name", sorted(FULL))
def test_gemm_full_size(torch_dev, orc, name):
    model, dt, gen = FULL[name]
    A, B, C = gen()
    say("full size", name)
    got, gx = run_gemm(torch_dev, model, dt, A, B, C)
    # the fingerprint is the XOR of each row of D
    assert np.array_equal(gx, np.bitwise_xor.reduce(got, axis=1))
    for r0, r1 in SAMPLE_ROWS:
        want, wx = orc.gemm_rows(model, dt, A, B, C, r0, r1)
        assert_bits_equal(got[r0:r1], want, f"{name} rows {r0}:{r1}")
        assert_bits_equal(gx[r0:r1], wx, f"{name} xorsum rows {r0}:{r1}")
    d = DIGESTS.get(name)
    assert d, f"no stored oracle digest for {name}"
    assert sha(got) == d["D_sha256"], f"{name}: D differs from the oracle's full output"
    assert sha(gx) == d["xorsum_sha256"], f"{name}: xorsum differs from the oracle's"
    if name == "gemm_4096_e4m3_hopper":
        # self-equivalence: recompute and compare the fingerprints and D
        say("full size recompute", name)
        got2, gx2 = run_gemm(torch_dev, model, dt, A, B, C)
        assert np.array_equal(gx2, gx) and np.array_equal(got2, got)


# --------------------------------------- the kernel that unpacks in place
@pytest.fixture
def no_workspace():
    """Force the tiled kernel's variant that needs no pre-pass workspace (the
    library reads MMAEMU_NO_WORKSPACE and MMAEMU_NARROW_BLOCKS on every call;
    0 keeps small shapes off the narrow kernel)."""
    os.environ["MMAEMU_NO_WORKSPACE"] = "1"
    os.environ["MMAEMU_NARROW_BLOCKS"] = "0"
    yield
    del os.environ["MMAEMU_NO_WORKSPACE"]
    del os.environ["MMAEMU_NARROW_BLOCKS"]


# MMAEMU_NARROW_BLOCKS replaces the library's kernel estimate by a
# block-count threshold (0: never the narrow kernel, a huge value: always,
# where it applies); MMAEMU_SPREAD_LANES then picks the narrow kernel itself
# (0) or the spread kernel with 2 or 4 lanes per output.
KERNEL_ENV = {
    "tiled": {"MMAEMU_NARROW_BLOCKS": "0"},
    "narrow": {"MMAEMU_NARROW_BLOCKS": str(1 << 40), "MMAEMU_SPREAD_LANES": "0"},
    # no workspace: the narrow kernel decodes A itself instead of copying
    # the pre-pass's row images
    "narrow-lds": {"MMAEMU_NARROW_BLOCKS": str(1 << 40), "MMAEMU_SPREAD_LANES": "0",
                   "MMAEMU_NO_WORKSPACE": "1"},
    "spread2": {"MMAEMU_NARROW_BLOCKS": str(1 << 40), "MMAEMU_SPREAD_LANES": "2"},
    "spread4": {"MMAEMU_NARROW_BLOCKS": str(1 << 40), "MMAEMU_SPREAD_LANES": "4"},
}


@pytest.fixture(params=list(KERNEL_ENV))
def gemm_kernel(request):
    """Run a test once on each GEMM kernel: the tiled one (4x4 outputs per
    lane), the narrow one (one output per lane) and the spread one (each
    output over 2 or 4 lanes), the last two of which the library takes for
    plain chains where it estimates them the faster."""
    env = KERNEL_ENV[request.param]
    os.environ.update(env)
    yield request.param
    for k in env:
        del os.environ[k]


@pytest.mark.parametrize("model,dt", COMBOS)
def test_gemm_in_place_unpack_path(torch_dev, orc, no_workspace, model, dt):
    for kind in ("normal", "wide", "specials"):
        for si, (M, N, K) in enumerate(SHAPES[2:]):
            A, B, C = _gen(kind, model, dt, M, N, K, 2000 + si)
            say("gemm (no workspace)", model, dt, kind, (M, N, K))
            got, gx = run_gemm(torch_dev, model, dt, A, B, C)
            want, wx = orc.gemm(model, dt, A, B, C)
            assert_bits_equal(got, want, f"gemm/no-ws {model}/{dt}/{kind} {M}x{N}x{K}")
            assert_bits_equal(gx, wx, f"gemm/no-ws xorsum {model}/{dt}/{kind} {M}x{N}x{K}")


def test_gemm_full_size_in_place_unpack_path(torch_dev, no_workspace):
    model, dt, gen = FULL["gemm_4096_fp16_ampere"]
    A, B, C = gen()
    say("full size (no workspace)", "gemm_4096_fp16_ampere")
    got, gx = run_gemm(torch_dev, model, dt, A, B, C)
    d = DIGESTS["gemm_4096_fp16_ampere"]
    assert sha(got) == d["D_sha256"] and sha(gx) == d["xorsum_sha256"]
