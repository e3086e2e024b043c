"""Seeded synthetic inputs for the emulated tile-MMA GEMM.

This module draws random numbers and casts them to the input formats; it
holds none of the emulated arithmetic, so the oracle side and the HIP side
can both consume its arrays.  Every array is a raw bit pattern:
uint16 codes for FP16/BF16, uint8 codes for FP8 E4M3 (OCP "FN" encoding),
uint32 patterns for the FP32 accumulator C.

The pages describe their workloads only as "10^5 random 16x16 tiles" and a
"4096x4096 MatMul" (Hawkeye reading notes, "Experiments and results"); the
concrete recipes below stand in for them:

  tiles_normal   A, B ~ N(0,1) in the format, C ~ N(0,1) FP32
  tiles_mixed    first half as tiles_normal, second half adversarial
                 (full exponent range, 5% subnormal and 1% zero elements,
                 exactly cancelling product pairs, Ampere stage-1 cancellation,
                 products near (2^p - 1)^2, C with wide exponents,
                 subnormals and zeros)
  gemm_normal    A, B ~ N(0,1) FP16, C = +0
  gemm_wide_bf16 A, B BF16 with random sign and magnitude 2^u, u ~ U(-60, 60),
                 rows i = 0 mod 16 of A scaled by 2^16; C ~ N(0,1)
  gemm_e4m3      A, B uniform over the 254 finite E4M3 codes; C ~ N(0,1)
"""
from __future__ import annotations

import numpy as np

FP16, BF16, E4M3 = 0, 1, 2
_CODE = {FP16: np.uint16, BF16: np.uint16, E4M3: np.uint8}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------- format casts
def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 codes of float32 values (round to nearest even)."""
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 codes of finite float32 values (round to nearest even)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def e4m3_finite_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform over the 254 finite E4M3FN codes (all but 0x7F and 0xFF)."""
    r = rng.integers(0, 254, size=shape, dtype=np.int32)
    r = r + (r >= 0x7F)
    return r.astype(np.uint8)


def normal_codes(rng, dtype: int, shape) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == FP16:
        return f32_to_fp16_bits(x)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError("normal_codes: FP16 or BF16 only")


# ------------------------------------------------------- format geometry
_GEOM = {FP16: (10, 5), BF16: (7, 8)}  # (fraction bits, exponent bits)


def _compose(sign, ef, frac, dtype):
    t, e = _GEOM[dtype]
    return ((sign.astype(np.uint32) << (t + e)) | (ef.astype(np.uint32) << t)
            | frac.astype(np.uint32)).astype(np.uint16)


def _adversarial_elements(rng, dtype, shape):
    """Sign uniform, exponent field uniform over the normal range with a
    uniform fraction; 5% subnormal (exponent field 0, non-zero fraction);
    1% signed zeros."""
    t, e = _GEOM[dtype]
    emax_field = (1 << e) - 2
    sign = rng.integers(0, 2, size=shape)
    ef = rng.integers(1, emax_field + 1, size=shape)
    frac = rng.integers(0, 1 << t, size=shape)
    u = rng.random(size=shape)
    sub = u < 0.05
    zero = (u >= 0.05) & (u < 0.06)
    ef = np.where(sub | zero, 0, ef)
    frac = np.where(sub, rng.integers(1, 1 << t, size=shape), frac)
    frac = np.where(zero, 0, frac)
    return _compose(sign, ef, frac, dtype)


def _adversarial_c(rng, dtype, shape):
    """50% N(0,1); 40% random sign with an FP32 exponent drawn uniformly over
    the format's product-exponent range clipped to FP32's normal range;
    5% FP32 subnormals; 5% signed zeros."""
    n = int(np.prod(shape))
    t, e = _GEOM[dtype]
    bias = (1 << (e - 1)) - 1
    pe_lo = max(2 * (1 - bias) - 2 * t, -126)
    pe_hi = min(2 * bias + 1, 127)
    out = f32_bits(rng.standard_normal(size=n, dtype=np.float32)).copy()
    u = rng.random(size=n)
    wide = (u >= 0.5) & (u < 0.9)
    sub = (u >= 0.9) & (u < 0.95)
    zero = u >= 0.95
    sign = rng.integers(0, 2, size=n).astype(np.uint32) << 31
    ef = (rng.integers(pe_lo, pe_hi + 1, size=n) + 127).astype(np.uint32)
    frac = rng.integers(0, 1 << 23, size=n).astype(np.uint32)
    out = np.where(wide, sign | (ef << 23) | frac, out)
    out = np.where(sub, sign | np.maximum(frac, 1), out)
    out = np.where(zero, sign, out)
    return out.astype(np.uint32).reshape(shape)


def _adversarial_tiles(rng, dtype, n):
    A = _adversarial_elements(rng, dtype, (n, 16, 16))
    B = _adversarial_elements(rng, dtype, (n, 16, 16))
    C = _adversarial_c(rng, dtype, (n, 16, 16))
    t, e = _GEOM[dtype]
    top = (1 << e) - 2
    kind = rng.random(size=n)
    # 5%: an exactly cancelling product pair, raised so that it sets emax
    for ti in np.nonzero(kind < 0.05)[0]:
        k1, k2 = rng.choice(16, size=2, replace=False)
        hi = rng.integers(top - 3, top + 1, size=2) if dtype == FP16 else \
            rng.integers(150, 190, size=2)
        A[ti, :, k1] = (A[ti, :, k1] & ~np.uint16(((1 << e) - 1) << t)) | np.uint16(hi[0] << t)
        B[ti, k1, :] = (B[ti, k1, :] & ~np.uint16(((1 << e) - 1) << t)) | np.uint16(hi[1] << t)
        B[ti, k2, :] = B[ti, k1, :]
        A[ti, :, k2] = A[ti, :, k1] ^ np.uint16(1 << (t + e))
    # 5%: Ampere stage-1 cancellation on half the rows: P2..P8 zeroed and
    # C = -P1 exactly (P1 kept inside FP32's normal range)
    for ti in np.nonzero((kind >= 0.05) & (kind < 0.10))[0]:
        bias = (1 << (e - 1)) - 1
        lo, hi = (1, top) if dtype == FP16 else (bias - 40, bias + 40)
        A[ti, :, 0] = _compose(rng.integers(0, 2, 16), rng.integers(lo, hi + 1, 16),
                               rng.integers(0, 1 << t, 16), dtype)
        B[ti, 0, :] = _compose(rng.integers(0, 2, 16), rng.integers(lo, hi + 1, 16),
                               rng.integers(0, 1 << t, 16), dtype)
        b = _decode_values(B[ti, 0, :], dtype)
        for i in range(0, 16, 2):
            A[ti, i, 1:8] = 0
            a = _decode_values(A[ti, i, 0:1], dtype)[0]
            C[ti, i, :] = f32_bits((-(a * b)).astype(np.float32))
    # 5%: every fraction all ones, exponents in a +-4 band
    for ti in np.nonzero((kind >= 0.10) & (kind < 0.15))[0]:
        bias = (1 << (e - 1)) - 1
        centre = rng.integers(bias - 6, bias + 7)
        for X in (A, B):
            s = rng.integers(0, 2, size=(16, 16))
            ef = np.clip(centre + rng.integers(-4, 5, size=(16, 16)), 1, top)
            X[ti] = _compose(s, ef, np.full((16, 16), (1 << t) - 1), dtype)
    return A, B, C


def _decode_values(codes, dtype) -> np.ndarray:
    """Exact float64 values of finite FP16/BF16 codes, via library casts."""
    codes = np.ascontiguousarray(codes, np.uint16)
    if dtype == FP16:
        return codes.view(np.float16).astype(np.float64)
    return (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# -------------------------------------------------------------- recipes
def tiles_normal(seed: int, ntiles: int, dtype: int = FP16):
    rng = _rng(seed)
    A = normal_codes(rng, dtype, (ntiles, 16, 16))
    B = normal_codes(rng, dtype, (ntiles, 16, 16))
    C = f32_bits(rng.standard_normal(size=(ntiles, 16, 16), dtype=np.float32))
    return A, B, C


def tiles_mixed(seed: int, ntiles: int, dtype: int):
    """First ntiles//2 tiles as tiles_normal, the rest adversarial."""
    rng = _rng(seed)
    h = ntiles // 2
    A1 = normal_codes(rng, dtype, (h, 16, 16))
    B1 = normal_codes(rng, dtype, (h, 16, 16))
    C1 = f32_bits(rng.standard_normal(size=(h, 16, 16), dtype=np.float32))
    A2, B2, C2 = _adversarial_tiles(rng, dtype, ntiles - h)
    return (np.concatenate([A1, A2]), np.concatenate([B1, B2]),
            np.concatenate([C1, C2]))


def gemm_normal(seed: int, M: int, N: int, K: int, dtype: int = FP16, c_zero: bool = True):
    rng = _rng(seed)
    A = normal_codes(rng, dtype, (M, K))
    B = normal_codes(rng, dtype, (K, N))
    if c_zero:
        C = np.zeros((M, N), np.uint32)
    else:
        C = f32_bits(rng.standard_normal(size=(M, N), dtype=np.float32))
    return A, B, C


def _log_uniform_bf16(rng, shape, lo=-60.0, hi=60.0):
    u = rng.uniform(lo, hi, size=shape)
    x = np.exp2(u) * np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    return f32_to_bf16_bits(x.astype(np.float32))


def gemm_wide_bf16(seed: int, M: int, N: int, K: int):
    rng = _rng(seed)
    A = _log_uniform_bf16(rng, (M, K))
    B = _log_uniform_bf16(rng, (K, N))
    # rows 0 mod 16: exponent field + 16 (exact scaling by 2^16; the
    # magnitudes stay below 2^77, far from the top of the BF16 range)
    rows = A[0::16].astype(np.uint32)
    nz = (rows & 0x7F80) != 0
    rows = np.where(nz, rows + (16 << 7), rows)
    A[0::16] = rows.astype(np.uint16)
    C = f32_bits(rng.standard_normal(size=(M, N), dtype=np.float32))
    return A, B, C


def gemm_e4m3(seed: int, M: int, N: int, K: int):
    rng = _rng(seed)
    A = e4m3_finite_codes(rng, (M, K))
    B = e4m3_finite_codes(rng, (K, N))
    C = f32_bits(rng.standard_normal(size=(M, N), dtype=np.float32))
    return A, B, C


def gemm_adversarial(seed: int, M: int, N: int, K: int, dtype: int, mode: str = "wide"):
    """Adversarial GEMM operands.  A, B start from the adversarial element mix
    (random sign, exponent field uniform over the normal range, 5% subnormal,
    1% signed zeros; for E4M3 the 254 finite codes); C from the adversarial
    FP32 mix.  mode:
      "wide"    as is (products span the whole range; BF16 chains overflow);
      "narrow"  normal exponents within +-3 of the bias: similar magnitudes;
      "coarse"  60% of the elements zero, the rest signed powers of two
                within +-1 of the bias, C a small signed power of two or
                zero: sums of few signed powers of two, which often cancel
                exactly;
      "tiny"    normal exponents in the lowest 6 binades and C among FP32
                subnormals and zeros: results near or below FP32's normal
                range."""
    rng = _rng(seed)
    if dtype == E4M3:
        A = e4m3_finite_codes(rng, (M, K))
        B = e4m3_finite_codes(rng, (K, N))
    else:
        A = _adversarial_elements(rng, dtype, (M, K))
        B = _adversarial_elements(rng, dtype, (K, N))
    C = _adversarial_c(rng, FP16 if dtype == E4M3 else dtype, (M, N))
    if mode == "wide":
        return A, B, C
    t, e = _GEOM[dtype] if dtype != E4M3 else (3, 4)
    bias = (1 << (e - 1)) - 1
    emask = np.uint32(((1 << e) - 1) << t)
    for X in (A, B):
        x = X.astype(np.uint32)
        ef = (x >> t) & ((1 << e) - 1)
        if mode == "narrow":
            band = (bias + rng.integers(-3, 4, size=X.shape)).astype(np.uint32)
        elif mode == "coarse":
            band = (bias + rng.integers(-1, 2, size=X.shape)).astype(np.uint32)
        else:  # tiny
            band = rng.integers(1, 7, size=X.shape).astype(np.uint32)
        x = np.where(ef != 0, (x & ~emask) | (band << t), x)
        if mode == "coarse":
            x = x & ~np.uint32((1 << t) - 1)     # signed powers of two (or zero)
            x = np.where(rng.random(X.shape) < 0.6, np.uint32(0), x)
        X[...] = x.astype(X.dtype)
    if mode == "coarse":
        pw = (127 + rng.integers(-2, 3, size=C.shape)).astype(np.uint32) << 23
        sg = rng.integers(0, 2, size=C.shape).astype(np.uint32) << 31
        C = np.where(rng.random(C.shape) < 0.5, sg | pw, sg).astype(np.uint32)
    elif mode == "tiny":
        fr = rng.integers(0, 1 << 23, size=C.shape).astype(np.uint32)
        sg = rng.integers(0, 2, size=C.shape).astype(np.uint32) << 31
        C = np.where(rng.random(C.shape) < 0.7, sg | fr, sg).astype(np.uint32)
    return A, B, C


def gemm_specials(seed: int, M: int, N: int, K: int, dtype: int):
    """Normal data sprinkled with inf, NaN, signed zeros and subnormals in A,
    B and C, to exercise the special-value rules (not a pages' workload)."""
    rng = _rng(seed)
    if dtype == E4M3:
        A = e4m3_finite_codes(rng, (M, K))
        B = e4m3_finite_codes(rng, (K, N))
        for X in (A, B):
            u = rng.random(X.shape)
            X[u < 0.002] = 0x7F
            X[(u >= 0.002) & (u < 0.004)] = 0xFF
            X[(u >= 0.004) & (u < 0.05)] = 0x80
    else:
        A = normal_codes(rng, dtype, (M, K))
        B = normal_codes(rng, dtype, (K, N))
        t, e = _GEOM[dtype]
        inf = np.uint16(((1 << e) - 1) << t)
        sbit = np.uint16(1 << (t + e))
        for X in (A, B):
            u = rng.random(X.shape)
            X[u < 0.001] = inf
            X[(u >= 0.001) & (u < 0.002)] = inf | sbit
            X[(u >= 0.002) & (u < 0.0025)] = inf | np.uint16(1)
            X[(u >= 0.0025) & (u < 0.05)] = sbit
            X[(u >= 0.05) & (u < 0.08)] = 0
            sub = (u >= 0.08) & (u < 0.12)
            X[sub] = (X[sub] & (sbit | np.uint16((1 << t) - 1))) | np.uint16(1)
    C = f32_bits(rng.standard_normal(size=(M, N), dtype=np.float32)).copy()
    u = rng.random(C.shape)
    C[u < 0.01] = 0x7F800000
    C[(u >= 0.01) & (u < 0.02)] = 0xFF800000
    C[(u >= 0.02) & (u < 0.025)] = 0x7FC00001
    C[(u >= 0.025) & (u < 0.06)] = 0x80000000
    C[(u >= 0.06) & (u < 0.1)] = 0x00000003
    return A, B, C


# -------------------------------------------------- the named workloads
WORKLOADS = {
    # name: (description, seed)
    "tiles_fp16_1k": ("1,000 independent 16x16x16 FP16 tiles, N(0,1), Ampere", 1001),
    "tiles_mixed_100k_fp16": ("100,000 FP16 tiles, half N(0,1), half adversarial", 2001),
    "tiles_mixed_100k_bf16": ("100,000 BF16 tiles, half N(0,1), half adversarial", 2002),
    "gemm_4096_fp16_ampere": ("GEMM 4096^3, FP16 N(0,1), C = 0, Ampere", 3001),
    "gemm_4096_bf16_hopper": ("GEMM 4096^3, BF16 log-uniform 2^+-60, scaled rows, Hopper", 4001),
    "gemm_4096_e4m3_hopper": ("GEMM 4096^3, E4M3 uniform finite codes, Hopper", 5001),
}
