"""The K-step order (mma_emulate_gemm_ordered) on the GPU against the
oracle's gemm_ordered, bit for bit: D and the per-row xorsum, on every
kernel that can run a chain (tiled with its pre-pass, tiled with its images
built in LDS, the narrow kernel, chunked workspaces), and at 4096^3 with the
256 steps reversed against the oracle's stored digest."""
import os

import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from test_gpu_parity import (COMBOS, DIGESTS, FULL, _gen, assert_bits_equal,  # noqa: F401
                             gemm_kernel, no_workspace, say, sha, to_dev, to_host_bits,
                             torch_dev)

pytestmark = pytest.mark.gpu


def _orders(rng, T):
    """Reversed, two random permutations, and a sequence with repeats and
    entries past the last step (read as T - 1)."""
    wild = rng.integers(0, T, size=T).astype(np.int64)
    wild[rng.integers(T)] = T + 5
    wild[rng.integers(T)] = -1
    return [np.arange(T - 1, -1, -1), rng.permutation(T), rng.permutation(T),
            wild.astype(np.int32)]


def run_ordered(torch_dev, model, dt, A, B, C, order, D=None):
    torch, dev = torch_dev
    tO = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).to(dev)
    D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B),
                   to_dev(torch_dev, C), D=D, xorsum=True, order=tO)
    return to_host_bits(D), to_host_bits(X)


@pytest.mark.parametrize("model,dt", COMBOS)
@pytest.mark.parametrize("kind", ["normal", "wide", "specials"])
def test_ordered_matches_oracle(torch_dev, orc, gemm_kernel, model, dt, kind):
    rng = np.random.default_rng(31)
    for si, (M, N, K) in enumerate([(17, 33, 48), (130, 100, 160), (3, 200, 256)]):
        A, B, C = _gen(kind, model, dt, M, N, K, 13000 + si)
        for order in _orders(rng, K // 16):
            say("ordered", gemm_kernel, model, dt, kind, (M, N, K), order.tolist())
            got, gx = run_ordered(torch_dev, model, dt, A, B, C, order)
            want, wx = orc.gemm_ordered(model, dt, A, B, C, order)
            what = f"ordered {gemm_kernel} {model}/{dt}/{kind} {M}x{N}x{K} {order.tolist()}"
            assert_bits_equal(got, want, what)
            assert_bits_equal(gx, wx, what + " xorsum")


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_ordered_without_workspace_and_in_place(torch_dev, orc, no_workspace, model, dt):
    rng = np.random.default_rng(32)
    M, N, K = 130, 100, 160
    A, B, C = _gen("specials", model, dt, M, N, K, 13100)
    for order in _orders(rng, K // 16):
        want, wx = orc.gemm_ordered(model, dt, A, B, C, order)
        say("ordered, images in LDS", model, dt, order.tolist())
        got, gx = run_ordered(torch_dev, model, dt, A, B, C, order)
        assert_bits_equal(got, want, f"ordered no-ws {model}/{dt} {order.tolist()}")
        assert_bits_equal(gx, wx, f"ordered no-ws xorsum {model}/{dt}")
        tC = to_dev(torch_dev, C)
        torch, dev = torch_dev
        tO = torch.from_numpy(order.astype(np.int32)).to(dev)
        D, X = mm.gemm(model, dt, to_dev(torch_dev, A), to_dev(torch_dev, B), tC, D=tC,
                       xorsum=True, order=tO)
        assert D.data_ptr() == tC.data_ptr()
        assert_bits_equal(to_host_bits(D), want, f"ordered in place {model}/{dt}")


def test_ordered_in_chunks(torch_dev, orc):
    """A workspace cap of 3 steps' images: the chain of 10 positions runs in
    chunks of 3, 3, 3 and 1, each pre-pass building its positions' images."""
    M, N, K = 130, 100, 160
    step_bytes = 12 * 1024 * (-(-M // 64) + -(-N // 64))
    os.environ["MMAEMU_NARROW_BLOCKS"] = "0"
    os.environ["MMAEMU_WORKSPACE_MAX_BYTES"] = str(3 * step_bytes)
    try:
        rng = np.random.default_rng(33)
        for model, dt in COMBOS:
            A, B, C = _gen("normal", model, dt, M, N, K, 13200)
            order = rng.permutation(10)
            say("ordered in chunks", model, dt, order.tolist())
            got, gx = run_ordered(torch_dev, model, dt, A, B, C, order)
            want, wx = orc.gemm_ordered(model, dt, A, B, C, order)
            assert_bits_equal(got, want, f"ordered chunks {model}/{dt}")
            assert_bits_equal(gx, wx, f"ordered chunks xorsum {model}/{dt}")
    finally:
        del os.environ["MMAEMU_NARROW_BLOCKS"]
        del os.environ["MMAEMU_WORKSPACE_MAX_BYTES"]


def test_forward_order_is_the_plain_chain(torch_dev, orc):
    M, N, K = 70, 90, 128
    A, B, C = _gen("wide", "hopper", "bf16", M, N, K, 13300)
    got, gx = run_ordered(torch_dev, "hopper", "bf16", A, B, C, np.arange(K // 16))
    want, wx = orc.gemm("hopper", "bf16", A, B, C)
    assert_bits_equal(got, want, "forward order")
    assert_bits_equal(gx, wx, "forward order xorsum")


def test_ordered_rejects_a_bad_order_tensor(torch_dev):
    torch, dev = torch_dev
    A = torch.zeros((16, 48), dtype=torch.int16, device=dev)
    B = torch.zeros((48, 16), dtype=torch.int16, device=dev)
    with pytest.raises(ValueError, match="order must have shape"):
        mm.gemm("ampere", "fp16", A, B, order=torch.zeros(2, dtype=torch.int32, device=dev))
    with pytest.raises(TypeError, match="int32"):
        mm.gemm("ampere", "fp16", A, B, order=torch.zeros(3, dtype=torch.int64, device=dev))
    with pytest.raises(ValueError, match="plain chain"):
        mm.gemm("ampere", "fp16", A, B, splits=3,
                order=torch.zeros(3, dtype=torch.int32, device=dev))


def test_ordered_full_size_reversed(torch_dev, orc):
    """4096^3 FP16 Ampere with the 256 K-steps reversed: the whole output
    against the oracle's stored digest, and sampled rows recomputed here."""
    model, dt, gen = FULL["gemm_4096_fp16_ampere"]
    A, B, C = gen()
    order = np.arange(255, -1, -1)
    say("ordered full size, reversed")
    got, gx = run_ordered(torch_dev, model, dt, A, B, C, order)
    for r0, r1 in [(0, 2), (2047, 2049), (4094, 4096)]:
        want, wx = orc.gemm_ordered(model, dt, A, B, C, order, rows=(r0, r1))
        assert_bits_equal(got[r0:r1], want, f"reversed full rows {r0}:{r1}")
        assert_bits_equal(gx[r0:r1], wx, f"reversed full xorsum rows {r0}:{r1}")
    d = DIGESTS["gemm_4096_fp16_ampere_reversed"]
    assert sha(got) == d["D_sha256"] and sha(gx) == d["xorsum_sha256"]
    # and it differs from the forward chain's output
    assert sha(got) != DIGESTS["gemm_4096_fp16_ampere"]["D_sha256"]
