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
