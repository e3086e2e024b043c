"""The allocation-free entry point (mma_emulate_gemm_noalloc_async) through
the C ABI against mma_emulate_gemm_async, bit for bit, on two calls in a
row, the second with a smaller input, so that the second call runs on what
the first left in the shared static scratch; at 4096^3 (a chain of 256
steps that runs in chunks of the scratch) also against the oracle's digest.
It must pass alone in a fresh process and after the other GPU tests."""
import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from test_gpu_parity import DIGESTS, FULL, _gen, say, sha, to_dev, torch_dev  # noqa: F401

pytestmark = pytest.mark.gpu

MODEL_ID = {"ampere": mm.AMPERE, "hopper": mm.HOPPER}
DT_ID = {"fp16": mm.FP16, "bf16": mm.BF16, "e4m3": mm.FP8_E4M3}


def _both(torch_dev, model, dt, A, B, C):
    """(D, xorsum) of the allocation-free call and of mma_emulate_gemm_async
    on the same inputs, as host bit arrays."""
    torch, dev = torch_dev
    M, K = A.shape
    N = B.shape[1]
    tA, tB, tC = to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C)
    outs = []
    for fn in (mm.mma_emulate_gemm_noalloc_async, mm.mma_emulate_gemm_async):
        D = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        X = torch.full((M,), -1, dtype=torch.int32, device=dev)
        s = torch.cuda.current_stream()
        rc = fn(MODEL_ID[model], DT_ID[dt], tA.data_ptr(), tB.data_ptr(),
                None if tC is None else tC.data_ptr(), D.data_ptr(), M, N, K, X.data_ptr(),
                s.cuda_stream)
        assert rc == 0, f"{fn.__name__}: {mm.mma_emulate_strerror(rc)}"
        torch.cuda.synchronize()
        outs.append((D.cpu().numpy().view(np.uint32), X.cpu().numpy().view(np.uint32)))
    return outs


def test_noalloc_full_size_then_smaller(torch_dev):
    """4096^3 FP16 Ampere (the oracle's digest too), then a smaller BF16
    Hopper GEMM with C on the same scratch."""
    model, dt, gen = FULL["gemm_4096_fp16_ampere"]
    A, B, C = gen()
    say("no-alloc 4096^3")
    (d1, x1), (d2, x2) = _both(torch_dev, model, dt, A, B, C)
    assert np.array_equal(d1, d2) and np.array_equal(x1, x2)
    d = DIGESTS["gemm_4096_fp16_ampere"]
    assert sha(d1) == d["D_sha256"] and sha(x1) == d["xorsum_sha256"]
    A, B, C = _gen("wide", "hopper", "bf16", 1000, 700, 512, 15000)
    say("no-alloc 1000x700x512 after it")
    (d1, x1), (d2, x2) = _both(torch_dev, "hopper", "bf16", A, B, C)
    assert np.array_equal(d1, d2) and np.array_equal(x1, x2)


def test_noalloc_small_shapes_in_a_row(torch_dev):
    """A tiled-kernel shape with specials, then a few-output shape (the
    spread kernel, its images in the scratch), then a smaller tiled one,
    each against the pooled call."""
    for model, dt, (M, N, K), kind in (("hopper", "e4m3", (300, 260, 640), "specials"),
                                       ("ampere", "fp16", (3, 900, 256), "normal"),
                                       ("ampere", "bf16", (130, 100, 160), "specials")):
        A, B, C = _gen(kind, model, dt, M, N, K, 15100 + M)
        say("no-alloc", model, dt, (M, N, K))
        (d1, x1), (d2, x2) = _both(torch_dev, model, dt, A, B, C)
        assert np.array_equal(d1, d2) and np.array_equal(x1, x2), (model, dt, M, N, K)


def test_noalloc_spread_chain_in_chunks(torch_dev):
    """256 x 256 x 65536 on the spread kernel: its images take 80 KiB per
    position, so the 64 MiB scratch holds 819 of the 4096 positions and the
    chain runs in five chunks through D, where the pooled call holds them
    all; then a smaller few-output GEMM on the same scratch."""
    from bit_exact_matrix_amd import inputs as I
    A, B, C = I.gemm_normal(15400, 256, 256, 65536, I.FP16, c_zero=False)
    say("no-alloc spread 256x256x65536")
    (d1, x1), (d2, x2) = _both(torch_dev, "ampere", "fp16", A, B, C)
    assert np.array_equal(d1, d2) and np.array_equal(x1, x2)
    A, B, C = _gen("specials", "hopper", "e4m3", 40, 50, 1024, 15500)
    say("no-alloc spread 40x50x1024 after it")
    (d1, x1), (d2, x2) = _both(torch_dev, "hopper", "e4m3", A, B, C)
    assert np.array_equal(d1, d2) and np.array_equal(x1, x2)


def test_noalloc_rejects_a_shape_beyond_its_scratch(torch_dev):
    """ceil(M/64) + ceil(N/64) > 5461 on the tiled kernel: MMAEMU_ERR_SCRATCH
    before anything is enqueued (fake, never-used addresses)."""
    A, B, C, D = 1 << 40, 2 << 40, 3 << 40, 4 << 40   # 1 TiB apart: no overlap
    rc = mm.mma_emulate_gemm_noalloc_async(0, 0, A, B, C, D, 200000, 200000, 64, None, None)
    assert rc == -9, mm.mma_emulate_strerror(rc)
    assert "scratch" in mm.mma_emulate_strerror(-9)
