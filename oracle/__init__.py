"""CPU oracle of the bit-exact tile-MMA emulation -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's ``cpu_baseline`` leg
may import this package.  It wraps ``liboracle.so`` (plain C, built from
``mma_oracle.c`` with gcc) through ctypes, taking and returning numpy arrays
of raw bit patterns.  It shares no code with the HIP library.

The arithmetic it follows is the Hawkeye recovered MMA model ("Hawkeye:
Reproducing GPU-Level Non-Determinism (MLSys 2026)" reading notes, sections
"Key observations" and "Recovered Ampere FP16 pipeline"); each rule is stated
and cited at the top of ``mma_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mma_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

AMPERE, HOPPER, LOVELACE = 0, 1, 2
FP16, BF16, E4M3 = 0, 1, 2

MODELS = {"ampere": AMPERE, "hopper": HOPPER, "lovelace": LOVELACE}
DTYPES = {"fp16": FP16, "bf16": BF16, "e4m3": E4M3}
CODE_DTYPE = {FP16: np.uint16, BF16: np.uint16, E4M3: np.uint8}


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C99 + pthreads)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-std=c99", "-D_DEFAULT_SOURCE", "-O2", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-pthread", SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None


def _bind(lib):
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mma_oracle_gemm.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64, vp, i32]
    lib.mma_oracle_gemm_rows.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, i64,
                                         i64, i64, vp, i32]
    lib.mma_oracle_tiles.argtypes = [i32, i32, vp, vp, vp, vp, i64, vp, i32]
    lib.mma_oracle_dots.argtypes = [i32, i32, vp, vp, vp, vp, i64]
    lib.mma_oracle_num_cpus.argtypes = []
    for f in (lib.mma_oracle_gemm, lib.mma_oracle_gemm_rows, lib.mma_oracle_tiles,
              lib.mma_oracle_dots, lib.mma_oracle_num_cpus):
        f.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _enum(v, table):
    return table[v] if isinstance(v, str) else int(v)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _codes(x, dtype):
    x = np.ascontiguousarray(x)
    want = CODE_DTYPE[dtype]
    if x.dtype != want:
        raise TypeError(f"expected {np.dtype(want).name} codes, got {x.dtype}")
    return x


def _bits32(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        x = x.view(np.uint32)
    if x.dtype != np.uint32:
        raise TypeError(f"expected uint32/float32 bit patterns, got {x.dtype}")
    return x


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (code {rc})")


def num_cpus() -> int:
    return _load().mma_oracle_num_cpus()


def gemm(model, dtype, A, B, C=None, nthreads=0, xorsum=True, lib=None):
    """D (uint32 bits, M x N) and per-row xorsum (or None) of the emulated GEMM."""
    lib = lib or _load()
    m, d = _enum(model, MODELS), _enum(dtype, DTYPES)
    A, B, C = _codes(A, d), _codes(B, d), _bits32(C)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2 and (C is None or C.shape == (M, N))
    D = np.empty((M, N), np.uint32)
    x = np.empty(M, np.uint32) if xorsum else None
    _check(lib.mma_oracle_gemm(m, d, _ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K,
                                   _ptr(x), int(nthreads)), "mma_oracle_gemm")
    return D, x


def gemm_splitk(model, dtype, A, B, C, splits, nthreads=0, lib=None):
    """The split-K schedule: the K/16 steps cut into `splits` runs of equal
    length; run r is the chained GEMM over its K range, from C for r = 0 and
    from +0 otherwise; D is the sum of the runs' FP32 results in run order,
    each addition IEEE binary32 round-to-nearest-even (numpy float32), with
    NaN results written as 0x7FC00000.  Returns (D bits, per-row xorsum).
    This schedule is a reading: the pages name split-K as a production
    schedule whose order they did not characterise (Hawkeye notes, "Critical
    Analysis" and Future work 4)."""
    M, K = A.shape
    T = K // 16
    assert splits >= 1 and K % 16 == 0 and (T % splits == 0 if K else splits == 1)
    per = 16 * (T // splits) if K else 0
    acc = None
    for r in range(splits):
        P, _ = gemm(model, dtype, A[:, r * per:(r + 1) * per], B[r * per:(r + 1) * per, :],
                    C if r == 0 else None, nthreads=nthreads, xorsum=False, lib=lib)
        if acc is None:
            acc = P
        else:
            with np.errstate(invalid="ignore", over="ignore"):
                s = acc.view(np.float32) + P.view(np.float32)
            acc = s.view(np.uint32).copy()
            acc[np.isnan(s)] = 0x7FC00000
    x = np.zeros(M, np.uint32)
    for j in range(acc.shape[1]):
        x ^= acc[:, j]
    return acc, x


def step_sequence(order, T):
    """The step that each position of the chain applies: position s takes
    step order[s], read as an unsigned 32-bit integer and clamped to T - 1
    (reading: the order is a model input that the pages leave open; a
    permutation of 0..T-1 is the intended use, and the clamp gives every
    other sequence of T words a defined meaning)."""
    order = np.asarray(order)
    assert order.shape == (T,), f"an order needs one entry per K-step ({T})"
    return np.minimum(order.astype(np.int64) & 0xFFFFFFFF, T - 1)


def gemm_ordered(model, dtype, A, B, C, order, nthreads=0, lib=None, rows=None):
    """The chained GEMM with its K-steps taken in a given order: C_0 = C,
    C_{s+1} = one MMA step of C_s with step t = order[s] of A and B (the
    16 columns A[:, 16t..16t+15] and rows B[16t..16t+15, :]), D = C_T for
    the T = K/16 steps.  The pages leave the order in which a library walks
    K open, as a schedule still to be characterised (Hawkeye notes,
    "Critical Analysis" and Future work 4); the forward order 0, 1, .., T-1
    is the plain gemm.  Written as the plain gemm on A and B with their
    K-blocks gathered in that order.  rows = (r0, r1) computes rows
    [r0, r1) only.  Returns (D bits, per-row xorsum)."""
    M, K = A.shape
    steps = step_sequence(order, K // 16)
    cols = (16 * steps[:, None] + np.arange(16)[None, :]).reshape(-1)
    if rows is not None:
        r0, r1 = rows
        A = A[r0:r1]
        C = None if C is None else C[r0:r1]
    return gemm(model, dtype, np.ascontiguousarray(A[:, cols]),
                np.ascontiguousarray(B[cols, :]), C, nthreads=nthreads, lib=lib)


def compare(D, D_claimed):
    """Bitwise comparison of an emulated D with a claimed one (both M x N
    bit patterns): (number of differing elements, smallest differing
    row-major index or None, per-row XOR of D ^ D_claimed as uint32[M])."""
    D = _bits32(D)
    claimed = _bits32(D_claimed)
    assert claimed.shape == D.shape
    diff = D ^ claimed
    bad = np.flatnonzero(diff)
    rows = np.zeros(D.shape[0], np.uint32)
    for j in range(D.shape[1]):
        rows ^= diff[:, j]
    return int(bad.size), (int(bad[0]) if bad.size else None), rows


def verify(model, dtype, A, B, C, D_claimed, nthreads=0, lib=None):
    """Audit compare, as the auditor of the Hawkeye notes does it ("Problem
    and motivation", "Relation to the verifiable-ML workflow"): recompute
    D = C + A.B with the characterised arithmetic and compare the provider's
    claimed D with it bit for bit.  Returns what ``compare`` returns."""
    D, _ = gemm(model, dtype, A, B, C, nthreads=nthreads, xorsum=False, lib=lib)
    return compare(D, D_claimed)


def gemm_rows(model, dtype, A, B, C, row_begin, row_end, nthreads=0, lib=None):
    """Rows [row_begin, row_end) of D and their xorsums."""
    lib = lib or _load()
    m, d = _enum(model, MODELS), _enum(dtype, DTYPES)
    A, B, C = _codes(A, d), _codes(B, d), _bits32(C)
    M, K = A.shape
    N = B.shape[1]
    rows = row_end - row_begin
    D = np.empty((rows, N), np.uint32)
    x = np.empty(rows, np.uint32)
    _check(lib.mma_oracle_gemm_rows(m, d, _ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K,
                                        row_begin, row_end, _ptr(x), int(nthreads)),
           "mma_oracle_gemm_rows")
    return D, x


def tiles(model, dtype, A, B, C=None, nthreads=0, lib=None):
    """D and per-tile xorsum of ntiles independent 16x16x16 MMAs."""
    lib = lib or _load()
    m, d = _enum(model, MODELS), _enum(dtype, DTYPES)
    A, B, C = _codes(A, d), _codes(B, d), _bits32(C)
    n = A.shape[0]
    assert A.shape == (n, 16, 16) and B.shape == (n, 16, 16)
    D = np.empty((n, 16, 16), np.uint32)
    x = np.empty(n, np.uint32)
    _check(lib.mma_oracle_tiles(m, d, _ptr(A), _ptr(B), _ptr(C), _ptr(D), n, _ptr(x),
                                    int(nthreads)), "mma_oracle_tiles")
    return D, x


def dots(model, dtype, a, b, c, lib=None):
    """d[r] = one MMA step for a single output: c[r] + sum_k a[r,k] b[r,k]."""
    lib = lib or _load()
    m, d = _enum(model, MODELS), _enum(dtype, DTYPES)
    a, b, c = _codes(a, d), _codes(b, d), _bits32(c)
    n = a.shape[0]
    assert a.shape == (n, 16) and b.shape == (n, 16) and c.shape == (n,)
    out = np.empty(n, np.uint32)
    _check(lib.mma_oracle_dots(m, d, _ptr(a), _ptr(b), _ptr(c), _ptr(out), n),
           "mma_oracle_dots")
    return out


class Library:
    """The same functions bound to another build of the oracle source (used
    by the tests that plant mistakes in a copy of it)."""

    def __init__(self, path):
        self.lib = _bind(ctypes.CDLL(path))

    def gemm(self, *a, **k):
        return gemm(*a, lib=self.lib, **k)

    def gemm_rows(self, *a, **k):
        return gemm_rows(*a, lib=self.lib, **k)

    def tiles(self, *a, **k):
        return tiles(*a, lib=self.lib, **k)

    def dots(self, *a, **k):
        return dots(*a, lib=self.lib, **k)


def build_library(src_path, out_path):
    """Compile an oracle source file (e.g. a modified copy) to out_path."""
    cmd = ["gcc", "-std=c99", "-D_DEFAULT_SOURCE", "-O1", "-fPIC", "-shared", "-w",
           "-pthread", "-I", HERE, src_path, "-o", out_path]
    subprocess.run(cmd, check=True)
    return Library(out_path)
