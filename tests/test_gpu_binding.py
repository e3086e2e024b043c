"""The torch layer of the binding on the GPU: calls on an explicit side
stream give the oracle's results (outputs are allocated under that stream),
and operand checks raise before any launch."""
import numpy as np
import pytest

import bit_exact_matrix_amd as mm
from bit_exact_matrix_amd import inputs as I
from test_gpu_parity import assert_bits_equal, say, to_dev, to_host_bits, torch_dev  # noqa: F401

pytestmark = pytest.mark.gpu


def test_side_stream_gemm_verify_and_tiles(torch_dev, orc):
    torch, dev = torch_dev
    side = torch.cuda.Stream(device=dev)
    A, B, C = I.gemm_normal(9600, 70, 90, 64, I.FP16, c_zero=False)
    want, wx = orc.gemm("ampere", "fp16", A, B, C)
    tA, tB, tC = to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C)
    side.wait_stream(torch.cuda.current_stream())   # the operands' copies are done
    say("side stream gemm / verify / tiles")
    D, X = mm.gemm("ampere", "fp16", tA, tB, tC, xorsum=True, stream=side)
    report, rows = mm.verify("ampere", "fp16", tA, tB, tC, D, row_diff=True, stream=side)
    At, Bt, Ct = I.tiles_normal(9601, 50)
    wt, wtx = orc.tiles("hopper", "fp16", At, Bt, Ct)
    tAt, tBt, tCt = to_dev(torch_dev, At), to_dev(torch_dev, Bt), to_dev(torch_dev, Ct)
    side.wait_stream(torch.cuda.current_stream())
    Dt, Xt = mm.tiles("hopper", "fp16", tAt, tBt, tCt, xorsum=True, stream=side)
    side.synchronize()
    assert_bits_equal(to_host_bits(D), want, "side-stream gemm")
    assert_bits_equal(to_host_bits(X), wx, "side-stream gemm xorsum")
    assert mm.mismatches(report) == (0, None) and not to_host_bits(rows).any()
    assert_bits_equal(to_host_bits(Dt), wt, "side-stream tiles")
    assert_bits_equal(to_host_bits(Xt), wtx, "side-stream tiles xorsum")


def test_operand_checks(torch_dev):
    torch, dev = torch_dev
    a = torch.zeros((32, 32), dtype=torch.int16, device=dev)
    with pytest.raises(TypeError, match="2-byte|1-byte"):
        mm.gemm("hopper", "e4m3", a, a)                  # E4M3 codes are one byte
    with pytest.raises(ValueError, match="contiguous"):
        mm.gemm("ampere", "fp16", a.t()[:, :16], a[:16])
    with pytest.raises(TypeError, match="device tensor"):
        mm.gemm("ampere", "fp16", a, a, C=torch.zeros((32, 32)))
    with pytest.raises(ValueError, match="shape"):
        mm.gemm("ampere", "fp16", a, a, C=torch.zeros((32, 31), device=dev))


def test_concurrent_calls_from_host_threads(torch_dev, orc):
    """Four host threads, each on its own stream, emulate different GEMMs
    (with the workspace, split-K runs side by side, and tiles) at the same
    time; every result must be the oracle's."""
    import threading
    torch, dev = torch_dev
    cases = []
    for i in range(4):
        A, B, C = I.gemm_normal(9650 + i, 130 + 17 * i, 150, 256, I.FP16, c_zero=False)
        want, wx = (orc.gemm("hopper", "fp16", A, B, C) if i % 2 == 0
                    else orc.gemm_splitk("hopper", "fp16", A, B, C, 4))
        cases.append((A, B, C, want, wx, 1 if i % 2 == 0 else 4))
    At, Bt, Ct = I.tiles_normal(9660, 333)
    wt, wtx = orc.tiles("ampere", "fp16", At, Bt, Ct)
    results, errors = {}, []

    def work(i):
        try:
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                A, B, C, _, _, splits = cases[i]
                tA, tB, tC = to_dev(torch_dev, A), to_dev(torch_dev, B), to_dev(torch_dev, C)
                for _ in range(5):
                    D, X = mm.gemm("hopper", "fp16", tA, tB, tC, xorsum=True, splits=splits,
                                   stream=s)
                    Dt, Xt = mm.tiles("ampere", "fp16", to_dev(torch_dev, At),
                                      to_dev(torch_dev, Bt), to_dev(torch_dev, Ct),
                                      xorsum=True, stream=s)
            s.synchronize()
            results[i] = (D, X, Dt, Xt)
        except Exception as e:     # reported in the main thread
            errors.append((i, repr(e)))

    say("concurrent host threads")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (_, _, _, want, wx, _) in enumerate(cases):
        D, X, Dt, Xt = results[i]
        assert_bits_equal(to_host_bits(D), want, f"thread {i} gemm")
        assert_bits_equal(to_host_bits(X), wx, f"thread {i} gemm xorsum")
        assert_bits_equal(to_host_bits(Dt), wt, f"thread {i} tiles")
        assert_bits_equal(to_host_bits(Xt), wtx, f"thread {i} tiles xorsum")
