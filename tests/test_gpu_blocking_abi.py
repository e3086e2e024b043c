"""The blocking entry points through the C ABI, on real device buffers,
against the oracle bit for bit: mma_emulate_gemm (the GEMM call of the
interface), mma_emulate_gemm_splitk, mma_emulate_gemm_ordered and
mma_verify_gemm.  Each enqueues on the null stream and synchronises before
it returns, so the results are read back with no further synchronisation.

Also the workspace contract: after a blocking call, and after an
asynchronous one followed by a synchronisation, the library's workspace
pool holds no device memory (mma_emulate_workspace_held)."""
import os

import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from test_gpu_parity import (COMBOS, DIGESTS, FULL, _gen, assert_bits_equal, say,  # noqa: F401
                             sha, to_dev, torch_dev)

pytestmark = pytest.mark.gpu

MODEL_ID = {"ampere": mm.AMPERE, "hopper": mm.HOPPER, "lovelace": mm.LOVELACE}
DT_ID = {"fp16": mm.FP16, "bf16": mm.BF16, "e4m3": mm.FP8_E4M3}
# ragged shapes: a narrow-kernel one (few outputs) and a tiled-kernel one
SHAPES = [(5, 300, 64), (37, 45, 96), (130, 100, 160)]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _bits(t):
    # the blocking calls have synchronised already; .cpu() adds nothing
    return t.cpu().numpy().view(np.uint32)


def _held():
    rc, held = mm.mma_emulate_workspace_held(0)
    assert rc == 0, mm.mma_emulate_strerror(rc)
    return held


def _buffers(torch_dev, A, B, C, M, N):
    torch, dev = torch_dev
    tA, tB, tC = to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C)
    D = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    X = torch.zeros(M, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return tA, tB, tC, D, X


@pytest.mark.parametrize("model,dt", COMBOS)
def test_blocking_gemm(torch_dev, orc, model, dt):
    for si, (M, N, K) in enumerate(SHAPES):
        for kind in ("normal", "specials"):
            A, B, C = _gen(kind, model, dt, M, N, K, 12000 + si)
            tA, tB, tC, D, X = _buffers(torch_dev, A, B, C, M, N)
            say("blocking mma_emulate_gemm", model, dt, kind, (M, N, K))
            rc = mm.mma_emulate_gemm(MODEL_ID[model], DT_ID[dt], _ptr(tA), _ptr(tB), _ptr(tC),
                                     _ptr(D), M, N, K, _ptr(X))
            assert rc == 0, mm.mma_emulate_strerror(rc)
            want, wx = orc.gemm(model, dt, A, B, C)
            what = f"blocking gemm {model}/{dt}/{kind} {M}x{N}x{K}"
            assert_bits_equal(_bits(D), want, what)
            assert_bits_equal(_bits(X), wx, what + " xorsum")
            assert _held() == 0, what + ": workspace held after a blocking call"


@pytest.mark.parametrize("model,dt", [("ampere", "fp16"), ("hopper", "bf16"),
                                      ("hopper", "e4m3")])
def test_blocking_splitk_ordered_and_verify(torch_dev, orc, model, dt):
    rng = np.random.default_rng(13)
    for si, (M, N, K) in enumerate(SHAPES):
        A, B, C = _gen("specials", model, dt, M, N, K, 12100 + si)
        T = K // 16
        # split-K, two runs
        tA, tB, tC, D, X = _buffers(torch_dev, A, B, C, M, N)
        say("blocking mma_emulate_gemm_splitk", model, dt, (M, N, K))
        rc = mm.mma_emulate_gemm_splitk(MODEL_ID[model], DT_ID[dt], _ptr(tA), _ptr(tB),
                                        _ptr(tC), _ptr(D), M, N, K, 2, _ptr(X))
        assert rc == 0, mm.mma_emulate_strerror(rc)
        want, wx = orc.gemm_splitk(model, dt, A, B, C, 2)
        assert_bits_equal(_bits(D), want, f"blocking split-K {model}/{dt} {M}x{N}x{K}")
        assert_bits_equal(_bits(X), wx, f"blocking split-K xorsum {model}/{dt} {M}x{N}x{K}")
        assert _held() == 0
        # a random step order
        torch, dev = torch_dev
        order = rng.permutation(T).astype(np.int32)
        tO = torch.from_numpy(order).to(dev)
        tA, tB, tC, D, X = _buffers(torch_dev, A, B, C, M, N)
        say("blocking mma_emulate_gemm_ordered", model, dt, (M, N, K), order.tolist())
        rc = mm.mma_emulate_gemm_ordered(MODEL_ID[model], DT_ID[dt], _ptr(tA), _ptr(tB),
                                         _ptr(tC), _ptr(D), M, N, K, _ptr(tO), _ptr(X))
        assert rc == 0, mm.mma_emulate_strerror(rc)
        want, wx = orc.gemm_ordered(model, dt, A, B, C, order)
        assert_bits_equal(_bits(D), want, f"blocking ordered {model}/{dt} {M}x{N}x{K}")
        assert_bits_equal(_bits(X), wx, f"blocking ordered xorsum {model}/{dt} {M}x{N}x{K}")
        assert _held() == 0
        # the audit compare against the oracle's D with two planted flips
        Dw, _ = orc.gemm(model, dt, A, B, C, xorsum=False)
        claimed = Dw.copy()
        claimed[M // 2, N - 1] ^= np.uint32(0x00010000)
        claimed[M - 1, 0] ^= np.uint32(0x80000000)
        want = orc.compare(Dw, claimed)
        tA, tB, tC, _, X = _buffers(torch_dev, A, B, C, M, N)
        tD = to_dev(torch_dev, claimed)
        report = torch.zeros(2, dtype=torch.int64, device=dev)
        torch.cuda.synchronize()
        say("blocking mma_verify_gemm", model, dt, (M, N, K))
        rc = mm.mma_verify_gemm(MODEL_ID[model], DT_ID[dt], _ptr(tA), _ptr(tB), _ptr(tC),
                                _ptr(tD), M, N, K, _ptr(report), _ptr(X))
        assert rc == 0, mm.mma_emulate_strerror(rc)
        count, first = (int(v) for v in report.cpu().tolist())
        assert (count, None if first == -1 else first) == want[:2]
        assert np.array_equal(_bits(X), want[2])
        assert _held() == 0


def test_blocking_gemm_full_size(torch_dev):
    """mma_emulate_gemm at 4096^3 FP16 Ampere against the oracle's digest of
    the whole output."""
    model, dt, gen = FULL["gemm_4096_fp16_ampere"]
    A, B, C = gen()
    M = N = K = 4096
    tA, tB, tC, D, X = _buffers(torch_dev, A, B, C, M, N)
    say("blocking mma_emulate_gemm 4096^3")
    rc = mm.mma_emulate_gemm(MODEL_ID[model], DT_ID[dt], _ptr(tA), _ptr(tB), _ptr(tC), _ptr(D),
                             M, N, K, _ptr(X))
    assert rc == 0, mm.mma_emulate_strerror(rc)
    d = DIGESTS["gemm_4096_fp16_ampere"]
    assert sha(_bits(D)) == d["D_sha256"] and sha(_bits(X)) == d["xorsum_sha256"]
    assert _held() == 0


def test_async_workspace_is_released_at_the_next_synchronisation(torch_dev, orc):
    """Three asynchronous calls that take a workspace (the tiled kernel),
    then one synchronisation: the pool holds nothing afterwards, and the
    results are the oracle's."""
    torch, dev = torch_dev
    os.environ["MMAEMU_NARROW_BLOCKS"] = "0"
    try:
        M, N, K = 300, 260, 256
        A, B, C = _gen("normal", "hopper", "fp16", M, N, K, 12200)
        tA, tB, tC = to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C)
        outs = []
        for _ in range(3):
            outs.append(mm.gemm("hopper", "fp16", tA, tB, tC, xorsum=True))
        torch.cuda.synchronize()
        say("workspace after three asynchronous calls and a synchronisation:", _held())
        assert _held() == 0
        want, wx = orc.gemm("hopper", "fp16", A, B, C)
        for D, X in outs:
            assert_bits_equal(_bits(D), want, "async gemm")
            assert_bits_equal(_bits(X), wx, "async gemm xorsum")
    finally:
        del os.environ["MMAEMU_NARROW_BLOCKS"]
