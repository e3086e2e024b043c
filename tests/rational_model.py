"""Second, independent statement of the MMA rounding model in exact rationals.

Used only by the tests, as a witness against the C oracle.  Where the oracle
works on integer significands and shift distances, this model works on exact
``Fraction`` values: a term is truncated toward zero to a multiple of the
grid 2^(emax - F), a normalisation keeps the top W bits of a value, and the
FP32 write-back keeps the top 24 bits (or whole multiples of 2^-149).  Input
values come from library casts (numpy float16, a 16-bit shift for bfloat16,
torch's float8_e4m3fn), not from bit-field parsing.

Rules follow the Hawkeye reading notes ("Hawkeye: Reproducing GPU-Level
Non-Determinism (MLSys 2026)"): products exact and unnormalised with nominal
exponent Ea+Eb ("Key observations" 1 and 3), grouping C+P1..P8 then +P9..P16
for Ampere and one 17-term group for Hopper ("Key observation 2"), internal
widths of 24 and 25 bits and truncation toward zero at alignment and at the
write-back ("Key observation 3"), overflow of the final cast to infinity
("Experiments and results").
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np

FP16, BF16, E4M3 = 0, 1, 2
EMIN = {FP16: -14, BF16: -126, E4M3: -6, "fp32": -126}


def _value_fp16(code):
    return float(np.array([code], np.uint16).view(np.float16)[0])


def _value_bf16(code):
    return float(np.array([int(code) << 16], np.uint32).view(np.float32)[0])


_E4M3_TABLE = None


def _value_e4m3(code):
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        import torch
        t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
        _E4M3_TABLE = [float(v) for v in t.tolist()]
    return _E4M3_TABLE[int(code)]


def _value_fp32(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) & 0xFFFFFFFF))[0]


_VALUE = {FP16: _value_fp16, BF16: _value_bf16, E4M3: _value_e4m3, "fp32": _value_fp32}


class Term:
    """kind in {'zero', 'finite', 'inf', 'nan'}; value exact; E nominal."""

    __slots__ = ("kind", "neg", "value", "E")

    def __init__(self, kind, neg, value=Fraction(0), E=0):
        self.kind, self.neg, self.value, self.E = kind, neg, value, E


def decode(fmt, code) -> Term:
    v = _VALUE[fmt](code)
    neg = math.copysign(1.0, v) < 0 if not math.isnan(v) else False
    if math.isnan(v):
        return Term("nan", False)
    if math.isinf(v):
        return Term("inf", neg)
    if v == 0.0:
        return Term("zero", neg)
    fr = Fraction(v)
    # nominal exponent: that of the leading bit for normal values, emin for
    # values below the normal range (subnormals are not renormalised)
    e = math.frexp(abs(v))[1] - 1
    return Term("finite", neg, fr, max(e, EMIN[fmt]))


def product(a: Term, b: Term) -> Term:
    neg = a.neg != b.neg
    kinds = {a.kind, b.kind}
    if "nan" in kinds or kinds == {"inf", "zero"}:
        return Term("nan", False)
    if "inf" in kinds:
        return Term("inf", neg)
    if "zero" in kinds:
        return Term("zero", neg)
    return Term("finite", neg, a.value * b.value, a.E + b.E)


def _trunc_to_grid(x: Fraction, g: Fraction) -> Fraction:
    q = abs(x) / g
    t = q.numerator // q.denominator
    return (t * g) if x >= 0 else -(t * g)


def group(terms, F):
    """Returns ('zero', neg) or ('value', V exact, emax)."""
    fin = [t for t in terms if t.kind == "finite"]
    if not fin:
        return ("zero", all(t.neg for t in terms))
    emax = max(t.E for t in fin)
    g = Fraction(2) ** (emax - F)
    V = sum((_trunc_to_grid(t.value, g) for t in fin), Fraction(0))
    if V == 0:
        return ("zero", False)
    return ("value", V, emax)


def _lead_exp(V: Fraction) -> int:
    """floor(log2 |V|) for a non-zero rational."""
    a = abs(V)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def norm_term(V: Fraction, W: int) -> Term:
    L = _lead_exp(V)
    q = Fraction(2) ** (L - W + 1)
    return Term("finite", V < 0, _trunc_to_grid(V, q), L)


def to_fp32_bits(V: Fraction) -> int:
    neg = V < 0
    a = abs(V)
    if a >= Fraction(2) ** 128:
        return 0xFF800000 if neg else 0x7F800000
    L = _lead_exp(V)
    q = Fraction(2) ** max(L - 23, -149)
    r = _trunc_to_grid(a, q)
    bits = struct.unpack("<I", struct.pack("<f", float(r)))[0]
    return bits | (0x80000000 if neg else 0)


def step(model, fmt, c_bits, a_codes, b_codes) -> int:
    """One MMA step for one output; model 0 = Ampere, 1 = Hopper."""
    C = decode("fp32", c_bits)
    P = [product(decode(fmt, a), decode(fmt, b)) for a, b in zip(a_codes, b_codes)]
    allt = [C] + P
    if any(t.kind == "nan" for t in allt):
        return 0x7FC00000
    infs = {t.neg for t in allt if t.kind == "inf"}
    if len(infs) == 2:
        return 0x7FC00000
    if infs:
        return 0xFF800000 if True in infs else 0x7F800000
    if model == 0:
        g1 = group([C] + P[:8], 23)
        if g1[0] == "zero":
            s1 = Term("zero", g1[1])
        else:
            s1 = norm_term(g1[1], 24)
        g = group([s1] + P[8:], 23)
    else:
        g = group([C] + P, 24)
    if g[0] == "zero":
        return 0x80000000 if g[1] else 0
    return to_fp32_bits(g[1])


def gemm(model, fmt, A, B, C):
    """Chained GEMM over K/16 steps (small sizes only)."""
    M, K = A.shape
    N = B.shape[1]
    D = np.zeros((M, N), np.uint32)
    for i in range(M):
        for j in range(N):
            c = int(C[i, j]) if C is not None else 0
            for t in range(K // 16):
                c = step(model, fmt, c, [int(x) for x in A[i, 16 * t:16 * t + 16]],
                         [int(x) for x in B[16 * t:16 * t + 16, j]])
            D[i, j] = c
    return D
