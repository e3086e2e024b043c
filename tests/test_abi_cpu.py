"""Host-side checks of libmmaemu.so that need no GPU: the library loads,
exports every entry point include/mmaemu.h declares, and rejects bad
arguments before anything is enqueued (no compute call is made here)."""
import os
import re

import pytest

import bit_exact_matrix_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mma_\w+)\s*\(", text, re.M))
    return names


def test_library_loads_and_exports_every_declared_symbol():
    lib = mm.load_library()
    declared = _declared()
    assert declared >= set(mm.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_strerror_and_version():
    assert mm.mma_emulate_spec_version() >= 1
    for code in range(-9, 1):
        assert isinstance(mm.mma_emulate_strerror(code), str)
    assert "unknown" in mm.mma_emulate_strerror(42)


# Fake, never-dereferenced device addresses: every call below must fail
# argument validation before any HIP call.
A, B, C, D, X = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


@pytest.mark.parametrize("args,code", [
    ((7, 0, A, B, C, D, 32, 32, 32, X), -1),           # unknown model
    ((0, 9, A, B, C, D, 32, 32, 32, X), -2),           # unknown dtype
    ((0, 2, A, B, C, D, 32, 32, 32, X), -3),           # E4M3 with Ampere
    ((2, 2, A, B, C, D, 32, 32, 32, X), -3),           # E4M3 with Lovelace
    ((3, 0, A, B, C, D, 32, 32, 32, X), -1),           # model 3 does not exist
    ((0, 0, A, B, C, D, 32, 32, 24, X), -4),           # K not a multiple of 16
    ((0, 0, A, B, C, D, -1, 32, 32, X), -4),           # negative M
    ((0, 0, A, B, C, D, 1 << 40, 1 << 40, 32, X), -4),  # size overflow
    ((0, 0, A, B, C, 0, 32, 32, 32, X), -5),           # NULL D
    ((0, 0, 0, B, C, D, 32, 32, 32, X), -5),           # NULL A with K > 0
    ((0, 0, A, B, C, A + 64, 32, 32, 32, X), -6),      # D overlaps A
    ((0, 0, A, B, C, C + 4, 32, 32, 32, X), -6),       # D partially overlaps C
    ((0, 0, A, B, C, D, 32, 32, 32, D + 8), -6),       # xorsum inside D
])
def test_gemm_argument_errors(args, code):
    assert mm.mma_emulate_gemm_async(*args, None) == code


# misaligned pointers (an element's worth off): MMAEMU_ERR_ALIGN before any launch
@pytest.mark.parametrize("args,code", [
    ((0, 0, A + 1, B, C, D, 32, 32, 32, X), -8),        # FP16 codes at an odd address
    ((1, 1, A, B + 1, C, D, 32, 32, 32, X), -8),        # BF16 codes at an odd address
    ((0, 0, A, B, C + 2, D, 32, 32, 32, X), -8),        # C not 4-byte aligned
    ((0, 0, A, B, C, D + 2, 32, 32, 32, X), -8),        # D not 4-byte aligned
    ((0, 0, A, B, C, D, 32, 32, 32, X + 2), -8),        # xorsum not 4-byte aligned
])
def test_gemm_alignment_errors(args, code):
    assert mm.mma_emulate_gemm_async(*args, None) == code
    assert mm.mma_emulate_gemm_splitk_async(*args[:9], 1, args[9], None) == code
    assert mm.mma_emulate_gemm_ordered_async(*args[:9], 0, args[9], None) == code


O = 0x70000000  # fake step-order address


@pytest.mark.parametrize("args,code", [
    ((7, 0, A, B, C, D, 32, 32, 32, O, X), -1),          # unknown model
    ((0, 2, A, B, C, D, 32, 32, 32, O, X), -3),          # E4M3 with Ampere
    ((0, 0, A, B, C, D, 32, 32, 24, O, X), -4),          # K not a multiple of 16
    ((0, 0, A, B, C, 0, 32, 32, 32, O, X), -5),          # NULL D
    ((0, 0, A, B, C, D, 32, 32, 32, O + 2, X), -8),      # order not 4-byte aligned
    ((0, 0, A, B, C, D, 32, 32, 32, D + 64, X), -6),     # order inside D (written)
    ((0, 0, A, B, C, D, 32, 32, 32, X + 4, X), -6),      # order inside the xorsum words
])
def test_ordered_argument_errors(args, code):
    assert mm.mma_emulate_gemm_ordered_async(*args, None) == code
    assert mm.mma_emulate_gemm_ordered(*args) == code


def test_ordered_order_may_overlap_the_inputs_and_is_unused_without_steps():
    # the order is read-only, like A, B and C; with K = 0 (no steps) or an
    # empty D it is never read, so its alignment does not matter either
    assert mm.mma_emulate_gemm_ordered_async(0, 0, A, B, C, D, 0, 32, 32, A, X, None) == 0
    assert mm.mma_emulate_gemm_ordered_async(0, 0, A, B, C, D, 0, 32, 32, O + 1, 0, None) == 0


def test_noalloc_argument_errors():
    """The allocation-free GEMM validates like mma_emulate_gemm_async, and
    rejects a chain whose one K-step of operand images exceeds its 64 MiB
    scratch (ceil(M/64) + ceil(N/64) > 5461 on the tiled kernel) with
    MMAEMU_ERR_SCRATCH, all before any HIP call."""
    f = mm.mma_emulate_gemm_noalloc_async
    assert f(7, 0, A, B, C, D, 32, 32, 32, X, None) == -1
    assert f(0, 2, A, B, C, D, 32, 32, 32, X, None) == -3
    assert f(0, 0, A, B, C, D, 32, 32, 24, X, None) == -4
    assert f(0, 0, A + 1, B, C, D, 32, 32, 32, X, None) == -8
    assert f(0, 0, A, B, C, A + 64, 32, 32, 32, X, None) == -6
    big = (1 << 40, 2 << 40, 3 << 40, 4 << 40)   # 1 TiB apart: no overlap
    assert f(0, 0, *big, 200000, 200000, 64, None, None) == -9
    assert f(1, 1, *big, 349441, 64, 16, None, None) == -9      # 5461 + 1 blocks of 64
    assert f(0, 0, 0, 0, 0, 0, 0, 200000, 64, 0, None) == 0      # nothing to compute
    assert "scratch" in mm.mma_emulate_strerror(-9)


def test_workspace_held_arguments():
    lib = mm.load_library()
    assert lib.mma_emulate_workspace_held(0, None) == -5
    rc, held = mm.mma_emulate_workspace_held(-1)
    assert rc == -7 and held == 0          # no such device (or no GPU at all)
    assert "mma_emulate_workspace_held" in mm.mma_emulate_strerror(-7)


def test_gemm_empty_is_a_no_op():
    # an empty D with no xorsum words to write: nothing is enqueued (with
    # M > 0 rows and N = 0 the M xorsum words are written, on the GPU)
    assert mm.mma_emulate_gemm_async(0, 0, A, B, C, D, 0, 32, 32, X, None) == 0
    assert mm.mma_emulate_gemm_async(1, 2, A, B, C, D, 32, 0, 32, 0, None) == 0


@pytest.mark.parametrize("args,code", [
    ((3, 0, A, B, C, D, 4, X), -1),
    ((0, 2, A, B, C, D, 4, X), -3),
    ((0, 0, A, B, C, D, -4, X), -4),
    ((0, 0, A, B, C, 0, 4, X), -5),
    ((0, 0, A, B, C, B, 4, X), -6),
    ((0, 0, A + 1, B, C, D, 4, X), -8),
    ((0, 0, A, B, C, D, 4, X + 2), -8),
])
def test_tiles_argument_errors(args, code):
    assert mm.mma_emulate_tiles(*args, None) == code


def test_tiles_empty_is_a_no_op():
    assert mm.mma_emulate_tiles(0, 0, A, B, C, D, 0, X, None) == 0


def test_in_place_c_equals_d_passes_validation_only():
    # D == C is allowed; with M = 0 nothing runs, so this checks the alias rule alone
    assert mm.mma_emulate_gemm_async(0, 0, A, B, C, C, 0, 16, 16, X, None) == 0


R = 0x60000000  # fake report address


@pytest.mark.parametrize("args,code", [
    ((7, 0, A, B, C, D, 32, 32, 32, R, X), -1),        # unknown model
    ((0, 2, A, B, C, D, 32, 32, 32, R, X), -3),        # E4M3 with Ampere
    ((0, 0, A, B, C, D, 32, 32, 24, R, X), -4),        # K not a multiple of 16
    ((0, 0, A, B, C, D, 32, 32, 32, 0, X), -5),        # NULL report
    ((0, 0, A, B, C, 0, 32, 32, 32, R, X), -5),        # NULL claimed D
    ((0, 0, A, 0, C, D, 32, 32, 32, R, X), -5),        # NULL B with K > 0
    ((0, 0, A, B, C, D, 32, 32, 32, D + 8, X), -6),    # report inside the claimed D
    ((0, 0, A, B, C, D, 32, 32, 32, R, A + 4), -6),    # row words inside A
    ((0, 0, A, B, C, D, 32, 32, 32, R, R + 8), -6),    # row words overlap the report
    ((0, 0, A, B, C, D, 32, 32, 32, C + 64, X), -6),   # report inside C
    ((0, 0, A, B, C, D, 32, 32, 32, R + 4, X), -8),    # report not 8-byte aligned
    ((0, 0, A, B, C, D + 1, 32, 32, 32, R, X), -8),    # claimed D not 4-byte aligned
    ((0, 0, A, B, C, D, 32, 32, 32, R, X + 1), -8),    # row words not 4-byte aligned
])
def test_verify_argument_errors(args, code):
    assert mm.mma_verify_gemm_async(*args, None) == code
    assert mm.mma_verify_gemm(*args) == code


def test_torch_wrappers_reject_host_tensors_before_any_launch():
    """The torch wrappers check their operands on the host: a CPU tensor, a
    non-matrix or mismatched inner dimensions raise before the library is
    called."""
    import torch
    a = torch.zeros((16, 16), dtype=torch.int16)
    with pytest.raises(TypeError, match="device tensor"):
        mm.gemm("ampere", "fp16", a, a)
    with pytest.raises(TypeError, match="device tensor"):
        mm.verify("hopper", "bf16", a, a, None, torch.zeros((16, 16)))
    with pytest.raises(TypeError, match="device tensor"):
        mm.tiles("ampere", "fp16", a.reshape(1, 16, 16), a.reshape(1, 16, 16))
    with pytest.raises(ValueError, match="matrices|inner"):
        mm._matrix_shapes(a.reshape(1, 16, 16), a)
    with pytest.raises(ValueError, match="inner dimensions"):
        mm._matrix_shapes(torch.zeros((16, 32)), torch.zeros((16, 16)))
    with pytest.raises(TypeError, match="B must be"):
        mm._matrix_shapes(a, a.numpy())


def test_torch_wrappers_reject_unknown_model_and_dtype_names():
    import torch
    a = torch.zeros((16, 16), dtype=torch.int16)
    with pytest.raises(ValueError, match="unknown model 'volta'"):
        mm.gemm("volta", "fp16", a, a)
    with pytest.raises(ValueError, match="unknown dtype 'fp32'"):
        mm.tiles("hopper", "fp32", a.reshape(1, 16, 16), a.reshape(1, 16, 16))
    with pytest.raises(ValueError, match="unknown model"):
        mm.verify("", "bf16", a, a, None, torch.zeros((16, 16)))
