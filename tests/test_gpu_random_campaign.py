"""A seeded random campaign over every GPU path, against the oracle.

Each case draws a model and format (Lovelace included), an input recipe
(the four adversarial modes, inputs sprinkled with specials, or plain
normal inputs), a ragged shape (by default up to 299 x 299 x 640), and a
path: the tiled kernel with its pre-pass, the tiled kernel building its
images in LDS, the narrow kernel, the split-K schedule (a random divisor of
the step count), a random K-step order (on one of the three chain kernels,
now and then with repeated or out-of-range entries), the audit compare (0
to 4 planted bit flips), or a batch of up to 1999 independent tiles.  Every output word, fingerprint and
report must equal the oracle's.  MMAEMU_CAMPAIGN_CASES sets the number of cases (2000 by
default; a run of 25,000 took about 4.5 minutes on one MI355X), and
MMAEMU_CAMPAIGN_MAX_MN and MMAEMU_CAMPAIGN_MAX_STEPS the shape bounds (300
and 40 by default); MMAEMU_CAMPAIGN_FIRST starts at another case index, so
that a long run can cover cases no earlier run drew.
"""
import os
import time

import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from bit_exact_matrix_amd import inputs as I
from test_gpu_parity import DT, say, to_dev, to_host_bits, torch_dev  # noqa: F401

pytestmark = pytest.mark.gpu

COMBOS = [("ampere", "fp16"), ("hopper", "fp16"), ("ampere", "bf16"), ("hopper", "bf16"),
          ("hopper", "e4m3"), ("lovelace", "fp16")]
RECIPES = ["wide", "narrow", "coarse", "tiny", "specials", "normal"]
PATHS = ["tiled", "tiled-in-lds", "narrow", "narrow-lds", "spread2", "spread4", "splitk",
         "ordered", "verify", "tiles"]
ENV = ("MMAEMU_NARROW_BLOCKS", "MMAEMU_NO_WORKSPACE", "MMAEMU_SPREAD_LANES")
# shape bounds: M, N below MAX_MN, K up to 16 * MAX_STEPS
MAX_MN = int(os.environ.get("MMAEMU_CAMPAIGN_MAX_MN", "300"))
MAX_STEPS = int(os.environ.get("MMAEMU_CAMPAIGN_MAX_STEPS", "40"))


def _set_path(path):
    for k in ENV:
        os.environ.pop(k, None)
    if path in ("tiled", "tiled-in-lds"):
        os.environ["MMAEMU_NARROW_BLOCKS"] = "0"
    if path in ("tiled-in-lds", "narrow-lds"):
        os.environ["MMAEMU_NO_WORKSPACE"] = "1"
    if path in ("narrow", "narrow-lds", "spread2", "spread4"):
        os.environ["MMAEMU_NARROW_BLOCKS"] = str(1 << 40)
        os.environ["MMAEMU_SPREAD_LANES"] = {"spread2": "2", "spread4": "4"}.get(path, "0")


def _gemm_inputs(seed, recipe, dt, M, N, K):
    if recipe == "specials":
        return I.gemm_specials(seed, M, N, K, DT[dt])
    if recipe == "normal":
        return (I.gemm_e4m3(seed, M, N, K) if dt == "e4m3"
                else I.gemm_normal(seed, M, N, K, DT[dt], c_zero=False))
    return I.gemm_adversarial(seed, M, N, K, DT[dt], recipe)


def _tile_inputs(seed, dt, n):
    if dt != "e4m3":
        return I.tiles_mixed(seed, n, DT[dt])
    A, B, C = I.gemm_e4m3(seed, 16 * n, 16, 16)
    return (A.reshape(n, 16, 16), np.ascontiguousarray(np.tile(B, (n, 1)).reshape(n, 16, 16)),
            C.reshape(n, 16, 16))


def _one_case(torch_dev, orc, case):
    """Returns a description of the case if the GPU differs from the oracle."""
    rng = np.random.default_rng(1_000_000 + case)
    model, dt = COMBOS[rng.integers(len(COMBOS))]
    recipe = RECIPES[rng.integers(len(RECIPES))]
    path = PATHS[rng.integers(len(PATHS))]
    M, N = int(rng.integers(1, MAX_MN)), int(rng.integers(1, MAX_MN))
    T = int(rng.integers(1, MAX_STEPS + 1))
    K = 16 * T
    seed = 2_000_000 + case
    _set_path(path)
    what = f"case {case}: {model}/{dt}/{recipe}/{path}"
    if path == "tiles":
        n = int(rng.integers(1, 2000))
        A, B, C = _tile_inputs(seed, dt, n)
        want, wx = orc.tiles(model, dt, A, B, C)
        D, X = mm.tiles(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                        to_dev(torch_dev, C), xorsum=True)
        ok = (np.array_equal(to_host_bits(D), want) and np.array_equal(to_host_bits(X), wx))
        return None if ok else f"{what} {n} tiles"
    A, B, C = _gemm_inputs(seed, recipe, dt, M, N, K)
    what += f" {M}x{N}x{K}"
    args = (to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C))
    if path == "verify":
        Dw, _ = orc.gemm(model, dt, A, B, C, xorsum=False)
        claimed = Dw.copy()
        for _ in range(int(rng.integers(0, 5))):
            r, c = int(rng.integers(M)), int(rng.integers(N))
            claimed[r, c] ^= np.uint32(1 << int(rng.integers(32)))
        want = orc.compare(Dw, claimed)
        report, X = mm.verify(model, dt, *args, to_dev(torch_dev, claimed), row_diff=True)
        ok = mm.mismatches(report) == want[:2] and np.array_equal(to_host_bits(X), want[2])
        return None if ok else what
    if path == "ordered":
        kernel = ("tiled", "tiled-in-lds", "narrow", "narrow-lds", "spread2",
                  "spread4")[rng.integers(6)]
        _set_path(kernel)
        order = rng.permutation(T)
        if rng.integers(4) == 0:
            order = rng.integers(-2, T + 3, size=T)
        order = order.astype(np.int32)
        what += f" on {kernel}, order {order.tolist()}"
        want, wx = orc.gemm_ordered(model, dt, A, B, C, order)
        torch, dev = torch_dev
        D, X = mm.gemm(model, dt, *args, xorsum=True, order=torch.from_numpy(order).to(dev))
        ok = np.array_equal(to_host_bits(D), want) and np.array_equal(to_host_bits(X), wx)
        return None if ok else what
    splits = 1
    if path == "splitk":
        divisors = [d for d in range(1, T + 1) if T % d == 0]
        splits = divisors[rng.integers(len(divisors))]
        want, wx = orc.gemm_splitk(model, dt, A, B, C, splits)
        what += f" splits {splits}"
    else:
        want, wx = orc.gemm(model, dt, A, B, C)
    D, X = mm.gemm(model, dt, *args, xorsum=True, splits=splits)
    ok = np.array_equal(to_host_bits(D), want) and np.array_equal(to_host_bits(X), wx)
    return None if ok else what


def test_random_campaign(torch_dev, orc):
    n = int(os.environ.get("MMAEMU_CAMPAIGN_CASES", "2000"))
    first = int(os.environ.get("MMAEMU_CAMPAIGN_FIRST", "0"))
    failures = []
    last = time.monotonic()
    try:
        for case in range(first, first + n):
            bad = _one_case(torch_dev, orc, case)
            if bad:
                failures.append(bad)
                say("campaign: differs from the oracle:", bad)
            # a progress line every 500 cases or 30 s, whichever comes first
            if (case - first) % 500 == 499 or time.monotonic() - last > 30:
                say(f"campaign: {case - first + 1} of {n} cases, {len(failures)} differ")
                last = time.monotonic()
    finally:
        for k in ENV:
            os.environ.pop(k, None)
    assert not failures, f"{len(failures)} of {n} cases differ; first: {failures[0]}"
