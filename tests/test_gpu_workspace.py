"""The cap on the operand-image workspace (MMAEMU_WORKSPACE_MAX_BYTES).

With a cap too small for the images of all K/16 steps, the library fills the
workspace one split-K run at a time, or cuts run 0 into chunks of steps that
restart from the D the previous chunk wrote, or builds the images in LDS.
Every such schedule must give the oracle's D and xorsum bit for bit."""
import os

import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from test_gpu_parity import (COMBOS, DIGESTS, FULL, _gen, assert_bits_equal,  # noqa: F401
                             say, sha, to_dev, to_host_bits, torch_dev)

pytestmark = pytest.mark.gpu

IMAGE_BYTES = 12 * 1024   # one operand image: a 64-row (or 64-column) block, one K-step


def step_bytes(M, N):
    """Workspace bytes for one K-step of images of every block of A and B."""
    return IMAGE_BYTES * (-(-M // 64) + -(-N // 64))


@pytest.fixture
def cap():
    """Sets the cap; small shapes stay on the tiled kernel (the narrow one
    takes no workspace)."""
    def set_cap(nbytes):
        os.environ["MMAEMU_WORKSPACE_MAX_BYTES"] = str(nbytes)
    os.environ["MMAEMU_NARROW_BLOCKS"] = "0"
    yield set_cap
    os.environ.pop("MMAEMU_WORKSPACE_MAX_BYTES", None)
    del os.environ["MMAEMU_NARROW_BLOCKS"]


def run(torch_dev, model, dt, A, B, C, splits=1, in_place=False):
    tC = to_dev(torch_dev, C)
    D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B), tC,
                   D=tC if in_place else None, xorsum=True, splits=splits)
    return to_host_bits(D), to_host_bits(X)


@pytest.mark.parametrize("model,dt", COMBOS)
def test_chunked_steps_match_the_oracle(torch_dev, orc, cap, model, dt):
    M, N, K = 130, 100, 160          # 3 + 2 blocks, 10 K-steps
    for kind in ("normal", "specials"):
        A, B, C = _gen(kind, model, dt, M, N, K, 9000)
        want, wx = orc.gemm(model, dt, A, B, C)
        # chunks of 1 step; 3+3+3+1; 4+4+2; 9+1; then all 10 at once
        for steps in (1, 3, 4, 9, 10):
            cap(steps * step_bytes(M, N))
            for in_place in (False, True):
                say("chunked", model, dt, kind, steps, "in place" if in_place else "")
                got, gx = run(torch_dev, model, dt, A, B, C, in_place=in_place)
                what = f"chunks of {steps} {model}/{dt}/{kind} in_place={in_place}"
                assert_bits_equal(got, want, what)
                assert_bits_equal(gx, wx, what + " xorsum")


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_split_k_under_a_cap(torch_dev, orc, cap, model, dt):
    """Two runs of 5 steps: a cap of 5 steps fills the workspace once per
    run; 3 steps cut run 0 into 3 + 2 and build run 1's images in LDS; a cap
    below one step builds every image in LDS."""
    M, N, K = 70, 90, 160
    A, B, C = _gen("specials", model, dt, M, N, K, 9100)
    want, wx = orc.gemm_splitk(model, dt, A, B, C, 2)
    for steps in (5, 3, 0):
        cap(steps * step_bytes(M, N))
        say("split-K under a cap", model, dt, steps)
        got, gx = run(torch_dev, model, dt, A, B, C, splits=2)
        assert_bits_equal(got, want, f"split-K 2, cap of {steps} steps, {model}/{dt}")
        assert_bits_equal(gx, wx, f"split-K 2, cap of {steps} steps, {model}/{dt} xorsum")


def test_verify_under_a_cap(torch_dev, orc, cap):
    """The audit compare has no D to chain through: under a cap it builds
    its images in LDS, with the same report."""
    M, N, K = 130, 100, 160
    A, B, C = _gen("normal", "hopper", "fp16", M, N, K, 9200)
    D, _ = orc.gemm("hopper", "fp16", A, B, C, xorsum=False)
    claimed = D.copy()
    claimed[7, 11] ^= np.uint32(0x2)
    claimed[100, 0] ^= np.uint32(0x80000000)
    want = orc.compare(D, claimed)
    cap(3 * step_bytes(M, N))
    say("verify under a cap")
    report, X = mm.verify("hopper", "fp16", to_dev(torch_dev, A), to_dev(torch_dev, B),
                          to_dev(torch_dev, C), to_dev(torch_dev, claimed), row_diff=True)
    assert mm.mismatches(report) == want[:2]
    assert np.array_equal(to_host_bits(X), want[2])


def test_full_size_in_chunks(torch_dev, cap):
    """4096^3 FP16 Ampere with a 100 MiB cap: chunks of 66, 66, 66 and 58
    steps (1.5 MiB of images per step), against the oracle's digest."""
    model, dt, gen = FULL["gemm_4096_fp16_ampere"]
    A, B, C = gen()
    cap(100 << 20)
    say("full size in chunks")
    got, gx = run(torch_dev, model, dt, A, B, C)
    d = DIGESTS["gemm_4096_fp16_ampere"]
    assert sha(got) == d["D_sha256"] and sha(gx) == d["xorsum_sha256"]
