"""Characterisation sweeps on an MMA unit: the Hawkeye Target Tests pointed at
a black box that computes one 16x16x16 step, D = C + A.B (Hawkeye notes,
"Core method": the Target Tests table and the neutral-subgroup test,
Algorithm 4).

Each probe builds dot products with exactly representable inputs, runs them
on the unit under test and classifies the bit patterns it returns:

  summation order        every subset S of {C, P1..P16} with two or more
                         members, engineered to cancel exactly versus zeroed:
                         S is neutral iff both give the same bits.  The
                         neutral sets that contain C form a chain; its
                         successive differences are the accumulation groups.
  internal precision     C = 2^c plus eight products 2^(c-k): the largest k
                         up to which every such sum is kept exactly is the
                         number of fraction bits F kept below the leading
                         exponent; W = F + 1.
  alignment rounding     two terms of +-0.75 grid units next to C: toward
                         zero, nearest, down or up.
  product normalisation  P1 = 1.5 * 1.5 (value 2.25, unnormalised exponent 0)
                         with a term one grid unit below: kept iff products
                         enter the max search unnormalised ("delayed").
  subnormal products     a product with a subnormal operand sets the group
                         maximum; a bit of C between the grid of its nominal
                         exponent and that of its true leading bit survives
                         iff the product is renormalised.

The unit under test is a ``dots`` callable: (a[n,16], b[n,16], c[n]) of raw
codes (c as FP32 bit patterns) -> d[n] FP32 bit patterns, d[r] = c[r] +
sum_k a[r,k] b[r,k] as one MMA step.  ``gpu_dots`` runs them on the GPU
emulator (16 dot products per tile, on its diagonal).  ``characterise``
returns the recovered model-table row.

    python -m bit_exact_matrix_amd.characterise --model ampere --dtype fp16
"""
from __future__ import annotations

import argparse
import json
import struct
import time
from fractions import Fraction

import numpy as np

# format: fraction bits t, exponent bits, bias, has infinities, code type
_FMT = {"fp16": (10, 5, 15, True, np.uint16),
        "bf16": (7, 8, 127, True, np.uint16),
        "e4m3": (3, 4, 7, False, np.uint8)}
_CODE_CACHE: dict = {}


def _finite_values(dtype):
    """{exact value: code} over every finite code of the format (+0 only)."""
    if dtype in _CODE_CACHE:
        return _CODE_CACHE[dtype]
    t, eb, bias, has_inf, _ = _FMT[dtype]
    emask = (1 << eb) - 1
    table = {}
    for code in range(1 << (1 + t + eb)):
        s = code >> (t + eb)
        ef = (code >> t) & emask
        fr = code & ((1 << t) - 1)
        if has_inf and ef == emask:
            continue
        if not has_inf and ef == emask and fr == (1 << t) - 1:
            continue  # E4M3 NaN
        if ef == 0:
            v = Fraction(fr, 1 << t) * Fraction(2) ** (1 - bias)
        else:
            v = Fraction((1 << t) + fr, 1 << t) * Fraction(2) ** (ef - bias)
        if s:
            v = -v
        if v == 0 and s:
            continue
        table.setdefault(v, code)
    _CODE_CACHE[dtype] = table
    return table


def code_of(dtype, v) -> int:
    """The code of the exactly representable value v (ValueError otherwise)."""
    table = _finite_values(dtype)
    v = Fraction(v)
    if v not in table:
        raise ValueError(f"{v} is not exactly representable in {dtype}")
    return table[v]


def emin(dtype) -> int:
    t, eb, bias, _, _ = _FMT[dtype]
    return 1 - bias


def fraction_bits(dtype) -> int:
    return _FMT[dtype][0]


def f32_bits(v) -> int:
    """FP32 bit pattern of the exactly representable value v."""
    v = Fraction(v)
    x = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    back = Fraction(struct.unpack("<f", struct.pack("<I", x))[0])
    if back != v:
        raise ValueError(f"{v} is not exactly representable in FP32")
    return x


def f32_value(bits: int):
    """Exact value of a finite FP32 bit pattern (None for inf/NaN)."""
    f = struct.unpack("<f", struct.pack("<I", int(bits)))[0]
    if f != f or f in (float("inf"), float("-inf")):
        return None
    return Fraction(f)


def factor(dtype, v):
    """Codes (a, b) of the format with a * b == v exactly, where a is a power
    of two or 1.5 times one; the most balanced such pair (ValueError if the
    format has none)."""
    v = Fraction(v)
    table = _finite_values(dtype)
    half = (v.numerator.bit_length() - v.denominator.bit_length()) // 2
    for d in sorted(range(-48, 49), key=abs):
        for m in (Fraction(1), Fraction(3, 2)):
            a = m * Fraction(2) ** (half + d)
            if a in table and v / a in table:
                return table[a], table[v / a]
    raise ValueError(f"no exact factorisation of {v} in {dtype}")


class _Batch:
    """Rows of dot products under construction (16 slots; zero codes)."""

    def __init__(self, dtype):
        self.dtype = dtype
        self.a, self.b, self.c = [], [], []

    def add(self, terms, c=0):
        """terms: {slot k (0-based): (a code, b code)}; c: FP32 bits."""
        ct = _FMT[self.dtype][4]
        a = np.zeros(16, ct)
        b = np.zeros(16, ct)
        for k, (x, y) in terms.items():
            a[k], b[k] = x, y
        self.a.append(a)
        self.b.append(b)
        self.c.append(c)
        return len(self.a) - 1

    def run(self, dots):
        d = dots(np.array(self.a), np.array(self.b), np.array(self.c, np.uint32))
        return np.asarray(d, np.uint32)


# ----------------------------------------------------------- the probes
def _neutral_batches(dtype):
    """The neutral-subgroup enumeration: for each subset, one engineered and
    one zeroed dot product."""
    t = fraction_bits(dtype)
    # cancelling products x^2 (x, 2x representable): 2^24, or 2^14 for E4M3
    big_e = 7 if dtype == "e4m3" else 12
    x = Fraction(2) ** big_e
    big = code_of(dtype, x)
    nbig = code_of(dtype, -x)
    nbig2 = code_of(dtype, -2 * x)
    # small products with low-order bits below the grid of the engineered
    # maximum (2^(2*big_e - W + 1)), so that it truncates them
    small_a = code_of(dtype, 1 + Fraction(1, 1 << t))
    small_b = code_of(dtype, (1 + Fraction(1, 1 << t)) * (Fraction(1, 64) if dtype == "e4m3" else 1))
    c_small = f32_bits(1 + Fraction(1, 1 << 23))
    xx = x * x
    eng, zer = _Batch(dtype), _Batch(dtype)
    subsets = []
    for mask in range(1 << 17):
        members = [i for i in range(17) if mask >> i & 1]
        if len(members) < 2:
            continue
        has_c = 0 in members
        prods = [i - 1 for i in members if i > 0]
        terms = {k: (small_a, small_b) for k in range(16)}
        n = len(prods)
        if has_c:
            total = 0
            for j, k in enumerate(prods):
                neg = j % 2 == 1
                terms[k] = (nbig if neg else big, big)
                total += -1 if neg else 1
            c_eng = f32_bits(-total * xx)
        else:
            if n % 2 == 0:
                for j, k in enumerate(prods):
                    terms[k] = (nbig if j % 2 else big, big)
            else:  # x + x - 2x, then cancelling pairs
                terms[prods[0]] = (big, big)
                terms[prods[1]] = (big, big)
                terms[prods[2]] = (nbig2, big)
                for j, k in enumerate(prods[3:]):
                    terms[k] = (nbig if j % 2 else big, big)
            c_eng = c_small
        eng.add(terms, c_eng)
        zterms = dict(terms)
        for k in prods:
            zterms[k] = (0, terms[k][1])
        zer.add(zterms, 0 if has_c else c_small)
        subsets.append(tuple(members))
    return subsets, eng, zer


def summation_order(dots, dtype):
    """Neutral subsets of {C=0, P1=1, ..., P16=16} and the accumulation groups
    they imply (the chain of neutral sets containing C)."""
    subsets, eng, zer = _neutral_batches(dtype)
    d1, d2 = eng.run(dots), zer.run(dots)
    neutral = sorted((s for s, x, y in zip(subsets, d1, d2) if x == y), key=len)
    chain = [set(s) for s in neutral if 0 in s]
    groups, seen = [], set()
    for s in chain:
        if seen and not seen <= s:
            return neutral, None   # not a chain: no pyramid structure recovered
        groups.append(sorted(s - seen))
        seen = s
    return neutral, groups


def internal_width(dots, dtype):
    """W = F + 1, F the largest k such that for every k' <= k eight products
    of 2^(c-k') next to C = 2^c are kept exactly (D = C + 8 * 2^(c-k')).
    Exactness, not mere change, is tested, so that a unit rounding up at the
    first dropped bit is not taken for a wider one.  None if the smallest k
    already loses bits, or if the sum stays exact up to the largest k whose
    terms still show in the FP32 result (a width beyond what this probe can
    see)."""
    c = 8 if dtype == "e4m3" else 0
    C = Fraction(2) ** c
    batch, ks = _Batch(dtype), list(range(16, 27))   # 8 * 2^(c-26) is one FP32 ulp of C
    for k in ks:
        pair = factor(dtype, Fraction(2) ** (c - k))
        batch.add({j: pair for j in range(8)}, f32_bits(C))
    d = batch.run(dots)
    F = None
    for k, bits in zip(ks, d):
        if f32_value(bits) != C + 8 * Fraction(2) ** (c - k):
            break
        F = k
    if F is None or F == ks[-1]:
        return None
    return F + 1


def alignment_rounding(dots, dtype, W):
    """How the alignment shift drops the bits below the group grid."""
    F = W - 1
    c = 8 if dtype == "e4m3" else 0
    g = Fraction(2) ** (c - F)
    C = Fraction(2) ** c
    batch = _Batch(dtype)
    for sgn in (1, -1):
        p = factor(dtype, sgn * Fraction(3, 4) * g)
        batch.add({0: p, 1: p}, f32_bits(C))
    d = [f32_value(x) for x in batch.run(dots)]
    pos = {C: "drop", C + 2 * g: "up"}.get(d[0])
    neg = {C: "drop", C - 2 * g: "down"}.get(d[1])
    return {("drop", "drop"): "toward zero", ("up", "down"): "nearest",
            ("drop", "down"): "down", ("up", "drop"): "up"}.get((pos, neg), "unknown")


def product_normalisation(dots, dtype, W):
    """'delayed' if a product enters the maximum search with its unnormalised
    exponent Ea + Eb, 'normalised first' if with its leading-bit exponent."""
    F = W - 1
    s = 8 if dtype == "e4m3" else 0
    h = Fraction(3, 2)
    p1 = (code_of(dtype, h * 2 ** s), code_of(dtype, h))        # 2.25 * 2^s, exponent s
    p2 = (code_of(dtype, -h * 2 ** s), code_of(dtype, 1))       # -1.5 * 2^s
    low = Fraction(2) ** (s - F)                                # one grid unit at exponent s
    p3 = factor(dtype, low)
    batch = _Batch(dtype)
    batch.add({0: p1, 1: p2, 2: p3}, 0)
    d = f32_value(batch.run(dots)[0])
    base = Fraction(3, 4) * 2 ** s
    return {base + low: "delayed", base: "normalised first"}.get(d, "unknown")


def subnormal_products(dots, dtype, W):
    """'not renormalised' if a product with a subnormal operand enters the
    maximum search with the nominal exponent emin + Eb, 'renormalised' if
    with its true leading bit."""
    F = W - 1
    t, e0 = fraction_bits(dtype), emin(dtype)
    B = {"fp16": 0, "bf16": 60, "e4m3": 0}[dtype]
    smin = Fraction(2) ** (e0 - t)
    p1 = (code_of(dtype, smin), code_of(dtype, Fraction(2) ** B))
    lead = Fraction(2) ** (e0 - t + B)                          # P1's value
    probe = Fraction(2) ** (e0 + B - F - 1)                     # between the two grids
    C = lead / 2 + probe
    batch = _Batch(dtype)
    batch.add({0: p1}, f32_bits(C))
    d = f32_value(batch.run(dots)[0])
    return {lead + lead / 2 + probe: "renormalised",
            lead + lead / 2: "not renormalised"}.get(d, "unknown")


def characterise(dots, dtype, neutral=True):
    """The model-table row the probes recover, with per-probe seconds (probe
    construction and classification included) and the seconds spent inside
    the unit under test."""
    inside = [0.0, 0]

    def timed(a, b, c, _dots=dots):
        t0 = time.perf_counter()
        d = _dots(a, b, c)
        inside[0] += time.perf_counter() - t0
        inside[1] += len(c)
        return d

    dots = timed
    out, sec = {}, {}
    t0 = time.perf_counter()
    W = internal_width(dots, dtype)
    sec["internal_width"] = time.perf_counter() - t0
    out["internal_width"] = W
    if W is not None:
        for name, fn in (("alignment_rounding", alignment_rounding),
                         ("product_normalisation", product_normalisation),
                         ("subnormal_products", subnormal_products)):
            t0 = time.perf_counter()
            out[name] = fn(dots, dtype, W)
            sec[name] = time.perf_counter() - t0
    if neutral:
        t0 = time.perf_counter()
        sets, groups = summation_order(dots, dtype)
        sec["summation_order"] = time.perf_counter() - t0
        out["neutral_sets"] = [list(s) for s in sets]
        out["groups"] = groups
    out["seconds"] = sec
    out["unit_seconds"] = inside[0]
    out["dot_products"] = inside[1]
    return out


def gpu_dots(model, dtype):
    """The GPU emulator as the unit under test: dot product r runs as output
    (r % 16, r % 16) of tile r // 16 through mma_emulate_tiles."""
    import torch

    from . import tiles

    def dots(a, b, c):
        n = a.shape[0]
        nt = (n + 15) // 16
        ct = a.dtype
        A = np.zeros((nt * 16, 16), ct)
        B = np.zeros((nt * 16, 16), ct)
        C = np.zeros((nt, 16, 16), np.uint32)
        A[:n], B[:n] = a, b
        A = A.reshape(nt, 16, 16)                     # row i of tile t: dot 16t+i
        B = B.reshape(nt, 16, 16).transpose(0, 2, 1)  # column i of tile t: dot 16t+i
        idx = np.arange(16)
        Cd = np.zeros(nt * 16, np.uint32)
        Cd[:n] = c
        C[:, idx, idx] = Cd.reshape(nt, 16)
        dev = torch.device("cuda:0")
        view = np.int8 if ct == np.uint8 else np.int16
        tA = torch.from_numpy(np.ascontiguousarray(A).view(view)).to(dev)
        tB = torch.from_numpy(np.ascontiguousarray(B).view(view)).to(dev)
        tC = torch.from_numpy(C.view(np.float32)).to(dev)
        D, _ = tiles(model, dtype, tA, tB, tC)
        torch.cuda.synchronize()
        Dh = D.cpu().numpy().view(np.uint32)
        return Dh[:, idx, idx].reshape(-1)[:n].copy()

    return dots


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--model", default="ampere", choices=["ampere", "hopper", "lovelace"])
    p.add_argument("--dtype", default="fp16", choices=sorted(_FMT))
    p.add_argument("--no-neutral", action="store_true",
                   help="skip the 131,054-subset summation-order enumeration")
    args = p.parse_args()
    res = characterise(gpu_dots(args.model, args.dtype), args.dtype,
                       neutral=not args.no_neutral)
    res.pop("neutral_sets", None)
    print(json.dumps({"model": args.model, "dtype": args.dtype, **res}))


if __name__ == "__main__":
    main()
