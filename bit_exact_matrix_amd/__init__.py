"""Python binding of libmmaemu.so, the MI355X bit-exact tile-MMA emulator.

Argument marshalling only: every step of the emulation runs in the HIP
kernels of libmmaemu.so (see include/mmaemu.h for the arithmetic and the
ABI).  PyTorch supplies device memory and the current stream.  There is no
CPU fallback: if the library is missing or no GPU is present, the calls
raise.

The raw C entry points are available under their own names (the
``EXPORTED`` tuple) and take integers (device pointers) exactly as the C
functions do; ``gemm``, ``verify`` and ``tiles`` wrap them for torch
tensors.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmmaemu.so")

AMPERE, HOPPER, LOVELACE = 0, 1, 2
FP16, BF16, FP8_E4M3 = 0, 1, 2
MODELS = {"ampere": AMPERE, "hopper": HOPPER, "lovelace": LOVELACE}
DTYPES = {"fp16": FP16, "bf16": BF16, "e4m3": FP8_E4M3, "fp8_e4m3": FP8_E4M3}
EXPORTED = ("mma_emulate_gemm", "mma_emulate_gemm_async", "mma_emulate_gemm_splitk",
            "mma_emulate_gemm_splitk_async", "mma_emulate_gemm_noalloc_async",
            "mma_emulate_gemm_ordered",
            "mma_emulate_gemm_ordered_async", "mma_verify_gemm", "mma_verify_gemm_async",
            "mma_emulate_tiles", "mma_emulate_workspace_held", "mma_emulate_strerror",
            "mma_emulate_spec_version")


class MmaEmuError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {mma_emulate_strerror(code)} (code {code})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmmaemu.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it first (__graft_entry__.build())")
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.mma_emulate_gemm.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64, vp]
        lib.mma_emulate_gemm_async.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64, vp, vp]
        lib.mma_emulate_gemm_splitk.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64, i64,
                                                vp]
        lib.mma_emulate_gemm_splitk_async.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64,
                                                      i64, vp, vp]
        lib.mma_emulate_gemm_noalloc_async.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64,
                                                       vp, vp]
        lib.mma_emulate_gemm_ordered.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64, vp,
                                                 vp]
        lib.mma_emulate_gemm_ordered_async.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64,
                                                       vp, vp, vp]
        lib.mma_emulate_workspace_held.argtypes = [i32, ctypes.POINTER(ctypes.c_uint64)]
        lib.mma_verify_gemm.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64, vp, vp]
        lib.mma_verify_gemm_async.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64, vp, vp,
                                              vp]
        lib.mma_emulate_tiles.argtypes = [i32, i32, vp, vp, vp, vp, i64, vp, vp]
        lib.mma_emulate_strerror.argtypes = [i32]
        lib.mma_emulate_strerror.restype = ctypes.c_char_p
        lib.mma_emulate_spec_version.argtypes = []
        for f in (lib.mma_emulate_gemm, lib.mma_emulate_gemm_async,
                  lib.mma_emulate_gemm_splitk, lib.mma_emulate_gemm_splitk_async,
                  lib.mma_emulate_gemm_noalloc_async,
                  lib.mma_emulate_gemm_ordered, lib.mma_emulate_gemm_ordered_async,
                  lib.mma_verify_gemm, lib.mma_verify_gemm_async, lib.mma_emulate_tiles,
                  lib.mma_emulate_workspace_held, lib.mma_emulate_spec_version):
            f.restype = i32
        _lib = lib
    return _lib


# ------------------------------------------------------- raw C entry points
def mma_emulate_gemm(model, dtype, A, B, C, D, M, N, K, xorsum_out):
    return load_library().mma_emulate_gemm(model, dtype, A, B, C, D, M, N, K, xorsum_out)


def mma_emulate_gemm_async(model, dtype, A, B, C, D, M, N, K, xorsum_out, hip_stream):
    return load_library().mma_emulate_gemm_async(model, dtype, A, B, C, D, M, N, K,
                                                 xorsum_out, hip_stream)


def mma_emulate_gemm_splitk(model, dtype, A, B, C, D, M, N, K, splits, xorsum_out):
    return load_library().mma_emulate_gemm_splitk(model, dtype, A, B, C, D, M, N, K, splits,
                                                  xorsum_out)


def mma_emulate_gemm_splitk_async(model, dtype, A, B, C, D, M, N, K, splits, xorsum_out,
                                  hip_stream):
    return load_library().mma_emulate_gemm_splitk_async(model, dtype, A, B, C, D, M, N, K,
                                                        splits, xorsum_out, hip_stream)


def mma_emulate_gemm_noalloc_async(model, dtype, A, B, C, D, M, N, K, xorsum_out, hip_stream):
    return load_library().mma_emulate_gemm_noalloc_async(model, dtype, A, B, C, D, M, N, K,
                                                         xorsum_out, hip_stream)


def mma_emulate_gemm_ordered(model, dtype, A, B, C, D, M, N, K, order, xorsum_out):
    return load_library().mma_emulate_gemm_ordered(model, dtype, A, B, C, D, M, N, K, order,
                                                   xorsum_out)


def mma_emulate_gemm_ordered_async(model, dtype, A, B, C, D, M, N, K, order, xorsum_out,
                                   hip_stream):
    return load_library().mma_emulate_gemm_ordered_async(model, dtype, A, B, C, D, M, N, K,
                                                         order, xorsum_out, hip_stream)


def mma_emulate_workspace_held(device):
    """(return code, bytes): the device memory the workspace pool of HIP
    device `device` holds right now."""
    v = ctypes.c_uint64(0)
    rc = load_library().mma_emulate_workspace_held(int(device), ctypes.byref(v))
    return rc, int(v.value)


def mma_verify_gemm(model, dtype, A, B, C, D_claimed, M, N, K, report, row_diff_out):
    return load_library().mma_verify_gemm(model, dtype, A, B, C, D_claimed, M, N, K, report,
                                          row_diff_out)


def mma_verify_gemm_async(model, dtype, A, B, C, D_claimed, M, N, K, report, row_diff_out,
                          hip_stream):
    return load_library().mma_verify_gemm_async(model, dtype, A, B, C, D_claimed, M, N, K,
                                                report, row_diff_out, hip_stream)


def mma_emulate_tiles(model, dtype, A, B, C, D, ntiles, xorsum_out, hip_stream):
    return load_library().mma_emulate_tiles(model, dtype, A, B, C, D, ntiles, xorsum_out,
                                            hip_stream)


def mma_emulate_strerror(code) -> str:
    return load_library().mma_emulate_strerror(int(code)).decode()


def mma_emulate_spec_version() -> int:
    return load_library().mma_emulate_spec_version()


# ------------------------------------------------------------ torch layer
def _enum(v, table, what):
    if isinstance(v, str):
        if v.lower() not in table:
            raise ValueError(f"unknown {what} {v!r}: one of {', '.join(sorted(table))}")
        return table[v.lower()]
    return int(v)


def _dev_ptr(t, what, nbytes_elem=None, device=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, the call runs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if nbytes_elem is not None and t.element_size() != nbytes_elem:
        raise TypeError(f"{what}: expected {nbytes_elem}-byte elements, got {t.dtype}")
    return t.data_ptr()


def _check_shape(t, shape, what):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _launch(A, stream):
    """The device of A (every operand must be there) and the launch stream:
    the given one, else that device's current stream.  The wrappers make
    the device current and allocate their outputs under the launch stream,
    so that torch's allocator ties them to the stream that writes them."""
    import torch
    if not isinstance(A, torch.Tensor) or not A.is_cuda:
        raise TypeError("A must be a device tensor")
    dev = A.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    if s.device != dev:
        raise ValueError(f"the stream is on {s.device}, the operands on {dev}")
    return dev, s


def _matrix_shapes(A, B):
    import torch
    if not isinstance(B, torch.Tensor):
        raise TypeError("B must be a device tensor")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be matrices")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    return M, N, K


def gemm(model, dtype, A, B, C=None, D=None, xorsum=False, stream=None, splits=1,
         order=None):
    """Emulated D = C + A.B on the current stream.

    A: M x K and B: K x N device tensors of raw codes (2-byte elements for
    FP16/BF16, 1-byte for E4M3).  C: optional M x N float32 (bit patterns).
    splits > 1 selects the split-K schedule (mma_emulate_gemm_splitk).
    order: optional int32 device tensor of K/16 entries, the K-step of each
    chain position (mma_emulate_gemm_ordered); not with splits > 1.
    Returns (D, xorsum): D float32 M x N, xorsum int32 of M words (bit
    patterns of the per-row XOR) or None.
    """
    import torch
    m, d = _enum(model, MODELS, "model"), _enum(dtype, DTYPES, "dtype")
    esz = 1 if d == FP8_E4M3 else 2
    dev, s = _launch(A, stream)
    M, N, K = _matrix_shapes(A, B)
    _check_shape(C, (M, N), "C")
    _check_shape(D, (M, N), "D")
    if order is not None:
        if int(splits) != 1:
            raise ValueError("a step order applies to the plain chain (splits = 1)")
        _check_shape(order, (K // 16,), "order")
        if order.dtype != torch.int32:
            raise TypeError("order must be an int32 tensor")
    with torch.cuda.device(dev), torch.cuda.stream(s):
        if D is None:
            D = torch.empty((M, N), dtype=torch.float32, device=dev)
        X = torch.empty(M, dtype=torch.int32, device=dev) if xorsum else None
        if order is not None:
            where = "mma_emulate_gemm_ordered_async"
            rc = mma_emulate_gemm_ordered_async(
                m, d, _dev_ptr(A, "A", esz, dev), _dev_ptr(B, "B", esz, dev),
                _dev_ptr(C, "C", 4, dev), _dev_ptr(D, "D", 4, dev), M, N, K,
                _dev_ptr(order, "order", 4, dev), _dev_ptr(X, "xorsum", None, dev),
                s.cuda_stream)
        else:
            where = "mma_emulate_gemm_splitk_async"
            rc = mma_emulate_gemm_splitk_async(
                m, d, _dev_ptr(A, "A", esz, dev), _dev_ptr(B, "B", esz, dev),
                _dev_ptr(C, "C", 4, dev), _dev_ptr(D, "D", 4, dev), M, N, K, int(splits),
                _dev_ptr(X, "xorsum", None, dev), s.cuda_stream)
    if rc != 0:
        raise MmaEmuError(rc, where)
    return D, X


def verify(model, dtype, A, B, C, D_claimed, row_diff=False, stream=None):
    """Audit compare: emulate D = C + A.B and compare it bit for bit with
    D_claimed (M x N float32, bit patterns) without storing it.

    Returns (report, row_diff) as device tensors, enqueued on the stream:
    report int64[2] = (number of differing elements, smallest differing
    row-major index or -1 when none; the C ABI's UINT64_MAX read as int64),
    row_diff int32 of M words (XOR over each row of emulated ^ claimed) or
    None.  ``mismatches(report)`` turns the report into Python ints.
    """
    import torch
    m, d = _enum(model, MODELS, "model"), _enum(dtype, DTYPES, "dtype")
    esz = 1 if d == FP8_E4M3 else 2
    dev, s = _launch(A, stream)
    M, N, K = _matrix_shapes(A, B)
    _check_shape(C, (M, N), "C")
    _check_shape(D_claimed, (M, N), "D_claimed")
    with torch.cuda.device(dev), torch.cuda.stream(s):
        report = torch.empty(2, dtype=torch.int64, device=dev)
        X = torch.empty(M, dtype=torch.int32, device=dev) if row_diff else None
        rc = mma_verify_gemm_async(
            m, d, _dev_ptr(A, "A", esz, dev), _dev_ptr(B, "B", esz, dev),
            _dev_ptr(C, "C", 4, dev), _dev_ptr(D_claimed, "D_claimed", 4, dev), M, N, K,
            _dev_ptr(report, "report", None, dev), _dev_ptr(X, "row_diff", None, dev),
            s.cuda_stream)
    if rc != 0:
        raise MmaEmuError(rc, "mma_verify_gemm_async")
    return report, X


def mismatches(report):
    """(count, first index or None) from a verify() report tensor."""
    count, first = (int(v) for v in report.cpu().tolist())
    return count, (None if first == -1 else first)


def tiles(model, dtype, A, B, C=None, D=None, xorsum=False, stream=None):
    """ntiles independent 16x16x16 MMAs: A, B [n,16,16] codes, C [n,16,16] f32."""
    import torch
    m, d = _enum(model, MODELS, "model"), _enum(dtype, DTYPES, "dtype")
    esz = 1 if d == FP8_E4M3 else 2
    dev, s = _launch(A, stream)
    if not isinstance(B, torch.Tensor):
        raise TypeError("B must be a device tensor")
    n = A.shape[0] if A.dim() == 3 else -1
    if tuple(A.shape) != (n, 16, 16) or tuple(B.shape) != (n, 16, 16):
        raise ValueError("A and B must be [ntiles, 16, 16]")
    _check_shape(C, (n, 16, 16), "C")
    _check_shape(D, (n, 16, 16), "D")
    with torch.cuda.device(dev), torch.cuda.stream(s):
        if D is None:
            D = torch.empty((n, 16, 16), dtype=torch.float32, device=dev)
        X = torch.empty(n, dtype=torch.int32, device=dev) if xorsum else None
        rc = mma_emulate_tiles(m, d, _dev_ptr(A, "A", esz, dev), _dev_ptr(B, "B", esz, dev),
                               _dev_ptr(C, "C", 4, dev), _dev_ptr(D, "D", 4, dev), n,
                               _dev_ptr(X, "xorsum", None, dev), s.cuda_stream)
    if rc != 0:
        raise MmaEmuError(rc, "mma_emulate_tiles")
    return D, X
