// gemm_fast.h -- LDS-tiled integer-VALU GEMM of the emulated tile MMA.
//
// Same arithmetic as step_generic (mmaemu_common.h; rules in
// include/mmaemu.h), reorganised for gfx950:
//
//  * a 256-lane workgroup owns a 64x64 block of D; each lane owns a 4x4
//    register tile and walks the K/16 chained MMA steps, carrying its 16
//    accumulators in registers in a decoded form (no FP32 pack/unpack per
//    step);
//  * each K-step the workgroup needs the 64x16 A slice and the 16x64 B slice
//    as "operand images" in LDS (double-buffered): A significands
//    pre-shifted onto the group grid, B significands signed, sign masks,
//    16-bit exponent codes and per-row / per-column sign bitmasks.  The
//    images are either built once per GEMM by a pre-pass into a workspace
//    and copied with direct global->LDS loads, or built in the kernel from
//    the raw codes when no workspace is available;
//  * exponents are 16-bit "negated biased" codes NE = bias - E, two per
//    register, paired by OUTPUT (rows 2r and 2r+1 of the lane tile): one
//    packed add gives the exponents of two products, one packed min keeps
//    the running maximum of two outputs (pass 1), and a saturating packed
//    add of NE - min + 0xFFE0 yields both alignment distances already
//    clamped to 31 in their low 5 bits (the shifter reads 5 bits);
//  * pass 2 per product: v_mad_i32_i24 forms the exact product in one's
//    complement of B's sign (b*a + sb = m ^ sb), an arithmetic shift by the
//    clamped distance truncates the MAGNITUDE toward zero
//    (asr(m ^ s, d) = (m >> d) ^ s), and v_xad_u32 applies A's sign and
//    accumulates; the +1 owed by every negative term is added once per
//    group as a popcount of the XOR of the two sign bitmasks;
//  * a group sum of zero gets the exponent code 0xFFFF (a saturating add of
//    the leading-zero count, which is all ones for zero): as an Ampere
//    stage-1 term it then takes no part in stage 2, as a final result it
//    fails the range check;
//  * every rare case -- a zero result, an FP32-subnormal result, an inf or
//    NaN operand -- fails a range check and the lane's tile is recomputed
//    for that step by step_generic from the raw codes.
#pragma once

#include "mmaemu_common.h"

namespace mmaemu {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

namespace fastk {

constexpr int BM = 64, BN = 64, NT = 256;
// 16-bit exponent codes.  Operand: NE = 0x2000 - E; zero operand 0x3000
// (E = -4096, below every real term); inf/NaN operand 0x0400 (E = 7168,
// above every real term so the result lands out of range).
constexpr uint32_t OP_BIAS = 0x2000, OP_ZERO = 0x3000, OP_SPECIAL = 0x0400;
// Terms (products, C, the Ampere stage-1 sum): NE = 0x4000 - E.
constexpr int T_BIAS = 0x4000;
constexpr uint32_t C_ZERO = 0x6000;  // E = -8192
constexpr uint32_t C_NAN = 0x2000;   // E = 8192: always recomputed
constexpr uint32_t C_INF = 0x3C00;   // E = 1024: dominates every product
// A fast-path result must have its leading-bit exponent in [-126, 2047];
// [128, 2047] is an FP32 overflow and becomes the inf state.
constexpr uint32_t NE_OK_LO = T_BIAS - 2047, NE_OK_SPAN = 2047 + 126;
constexpr uint32_t NE_OVF = T_BIAS - 128;
// Term codes at or below this: a product with an inf/NaN operand (E >= 3072),
// or the NaN state; every real term lies far above it.
constexpr uint32_t SPECIAL_MAX = 0x3400;
constexpr unsigned short SAT = 0xFFE0;
// The code that rows of A and columns of B beyond the matrix read: 1.0.  A
// live output never reads them; a padding output then sums finite products
// and stays in range, so that ragged edge blocks do not take the exact
// recompute every step (with +0 codes their sums would fall out of range).
template <int DT>
constexpr uint32_t PAD_CODE = (uint32_t)Fmt<DT>::bias << Fmt<DT>::t;

// One operand's slice for one K-step, exactly as the consumer reads it from
// LDS.  Rows are padded from 64 to 68 words: writers store 16-byte chunks
// from lanes that differ in k, which would otherwise all hit the same banks;
// 68 keeps every row 16-byte aligned for the b128 reads.  The image is
// 12 KiB so that it can also be copied from HBM in whole 1 KiB wave loads.
//   ne, A image: word [p][2q + j] = NE of rows (2q, 2q+1) at k = 2p + j
//   ne, B image: word [p][c]      = NE of column c at k = 2p | k = 2p+1
constexpr int PAD = BM + 4;
constexpr int IMG_WORDS = 3072;
struct OpImage {
  uint32_t val[16][PAD];  // A: significand << (F - 2t); B: signed significand
  int32_t sgn[16][PAD];   // 0 / -1
  uint32_t ne[8][PAD];    // exponent codes, two per word (see above)
  uint32_t msk[2][PAD];   // sign bits of the row's / column's group products
  uint32_t pad_[IMG_WORDS - 42 * PAD];
};
static_assert(sizeof(OpImage) == 4 * IMG_WORDS, "operand image must be 12 KiB");
struct Stage {
  OpImage a, b;
};

__device__ __forceinline__ u16x2 as2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t as32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ u16x2 splat_lo(uint32_t x) {
  return u16x2{(unsigned short)x, (unsigned short)x};
}
__device__ __forceinline__ u16x2 splat_hi(uint32_t x) {
  return u16x2{(unsigned short)(x >> 16), (unsigned short)(x >> 16)};
}
__device__ __forceinline__ unsigned short half16(uint32_t x, int h) {
  return (unsigned short)(h ? x >> 16 : x);
}
// Leading zeros of x, and 0xFFFFFFFF for x = 0 (v_ffbh_u32 as is: __clz
// would add a clamp for the zero case).
__device__ __forceinline__ uint32_t ffbh(uint32_t x) {
  uint32_t r;
  asm("v_ffbh_u32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// The leading zeros of x (0xFFFF for x = 0) into the high word of packed,
// whose low word is kept: an SDWA v_ffbh_u32, so that a pair of counts
// needs no separate packing instruction.
__device__ __forceinline__ uint32_t ffbh_into_hi(uint32_t packed, uint32_t x) {
  asm("v_ffbh_u32_sdwa %0, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
      : "+v"(packed)
      : "v"(x));
  return packed;
}
// v_ffbh_i32: the count of leading bits equal to the sign bit, 0xFFFFFFFF
// for x = 0 (and -1).  For x = |S| ^ s (s = 0 or -1, S != -2^31) that is the
// leading zeros of |S|: the bits of ~|S| above |S|'s leading one are ones.
__device__ __forceinline__ uint32_t ffbh_i32(int x) {
  uint32_t r;
  asm("v_ffbh_i32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// The same count for x into the high word of packed (0xFFFF for x = 0).
__device__ __forceinline__ uint32_t ffbh_i32_into_hi(uint32_t packed, int x) {
  asm("v_ffbh_i32_sdwa %0, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
      : "+v"(packed)
      : "v"(x));
  return packed;
}
// Minimum of three pairs of 16-bit exponent codes.  Every code that reaches
// it is a positive normal binary16 bit pattern (0x0800 .. 0x6000), and for
// those the binary16 order is the integer order, so the packed binary16
// minimum3 folds two products' exponents per instruction.
__device__ __forceinline__ u16x2 min3h(u16x2 a, u16x2 b, u16x2 c) {
  uint32_t r;
  asm("v_pk_minimum3_f16 %0, %1, %2, %3" : "=v"(r) : "v"(as32(a)), "v"(as32(b)), "v"(as32(c)));
  return as2(r);
}
// (a ^ b) + c in one VALU op (the compiler prefers xor + add3 pairs).
__device__ __forceinline__ int xad(int a, int b, int c) {
  int r;
  asm("v_xad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// One operand: significand, sign mask, 16-bit exponent code.
template <int DT>
__device__ __forceinline__ void unpack(uint32_t code, uint32_t& m, int& s, uint32_t& ne) {
  using F = Fmt<DT>;
  constexpr uint32_t fmask = (1u << F::t) - 1u;
  constexpr uint32_t emask = (1u << F::eb) - 1u;
  const uint32_t frac = code & fmask;
  const uint32_t ef = (code >> F::t) & emask;
  s = -(int)((code >> (F::t + F::eb)) & 1u);
  const bool special = F::has_inf ? (ef == emask) : (ef == emask && frac == fmask);
  const bool sub = ef == 0;
  m = sub ? frac : (frac | (1u << F::t));
  const int E = sub ? 1 - F::bias : (int)ef - F::bias;
  ne = special ? OP_SPECIAL : (m == 0 ? OP_ZERO : (uint32_t)((int)OP_BIAS - E));
  // Zero and inf/NaN operands carry a dummy nonzero significand.  A product
  // with a zero operand sits thousands of binades below every real term, so
  // it is always shifted out, and a group made of nothing else lands out of
  // range.  A product with an inf/NaN operand (inf * 0 included) then never
  // sums to exactly zero: its huge exponent cannot be mistaken for an empty
  // Ampere stage-1 sum and always reaches the range check.
  if (special || m == 0) m = 1u << F::t;
}

// Accumulator state <-> FP32 bits.  X = M ^ s with M the significand on
// the group grid (24 bits, << (F-23)); ne = 0x4000 - E (16 bits).
template <int MODEL>
__device__ __forceinline__ void bits_to_state(uint32_t bits, int& X, uint32_t& ne) {
  constexpr int F = Model<MODEL>::F;
  const int s = (int)bits >> 31;
  const uint32_t ef = (bits >> 23) & 0xFFu, fr = bits & 0x7FFFFFu;
  uint32_t m;
  if (ef == 0xFFu) {
    m = 0x800000u;
    ne = fr ? C_NAN : C_INF;
  } else if (ef == 0) {
    m = fr;  // subnormal: exponent -126, not renormalised
    ne = fr ? (uint32_t)(T_BIAS + 126) : C_ZERO;
  } else {
    m = fr | 0x800000u;
    ne = (uint32_t)(T_BIAS - ((int)ef - 127));
  }
  X = (int)(m << (F - 23)) ^ s;
}

template <int MODEL>
__device__ __forceinline__ uint32_t state_to_bits(int X, uint32_t ne) {
  constexpr int F = Model<MODEL>::F;
  const int s = X >> 31;
  const uint32_t sign = (uint32_t)s & 0x80000000u;
  const uint32_t m = (uint32_t)(X ^ s) >> (F - 23);
  ne &= 0xFFFFu;
  if (ne == C_NAN) return kNaN;
  if (ne == C_ZERO) return sign;
  const int E = T_BIAS - (int)ne;
  if (E >= 128) return sign | kPosInf;
  if (m < 0x800000u) return sign | m;  // FP32 subnormal (E = -126)
  return sign | ((uint32_t)(E + 127) << 23) | (m & 0x7FFFFFu);
}

// Recompute one output's step from the raw codes in global memory (rare
// path): output (r, c) of the calling lane's 4x4 tile in the workgroup's
// 64x64 block, at chain position pos (the step order maps it to a K-step).  Rows and columns outside the matrix read the code of 1.0
// (PAD_CODE), as in the image builders.  The row and column are derived
// here rather than passed, so that the caller keeps no per-lane 64-bit
// indices live across its loop.
template <int MODEL, int DT>
__device__ __noinline__ uint2 slow_step(const void* A, const void* B, int64_t M, int64_t N,
                                        int64_t K, const int32_t* order, int64_t pos, int tr,
                                        int tc, int Xold, uint32_t ne_old) {
  const int64_t s = step_at(order, pos, K / 16);
  const int64_t row = (int64_t)blockIdx.y * BM + 4 * (threadIdx.x >> 4) + tr;
  const int64_t col = (int64_t)blockIdx.x * BN + 4 * (threadIdx.x & 15) + tc;
  uint32_t a[16], b[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    a[k] = row < M ? load_code<DT>(A, row * K + 16 * s + k) : PAD_CODE<DT>;
    b[k] = col < N ? load_code<DT>(B, (16 * s + k) * N + col) : PAD_CODE<DT>;
  }
  const uint32_t c = state_to_bits<MODEL>(Xold, ne_old);
  const uint32_t r = step_generic<MODEL, DT>(c, a, b);
  int X;
  uint32_t ne;
  bits_to_state<MODEL>(r, X, ne);
  return make_uint2((uint32_t)X, ne);
}

// Operand image contents of one element, A side and B side.
template <int MODEL, int DT>
__device__ __forceinline__ void image_a(uint32_t code, uint32_t& val, int& sgn, uint32_t& ne) {
  constexpr int pshift = Model<MODEL>::F - 2 * Fmt<DT>::t;
  uint32_t m;
  unpack<DT>(code, m, sgn, ne);
  val = m << pshift;
}
template <int DT>
__device__ __forceinline__ void image_b(uint32_t code, uint32_t& val, int& sgn, uint32_t& ne) {
  uint32_t m;
  unpack<DT>(code, m, sgn, ne);
  val = (uint32_t)(sgn ? -(int)m : (int)m);
}

// In-kernel image builder (no workspace): lane (k = t & 15, q = t >> 4)
// handles A rows 4q..4q+3 and B cols 4q..4q+3 at k.
template <int MODEL, int DT, typename ST>
__device__ __forceinline__ void produce(ST* st, const uint32_t (&ca)[4],
                                        const uint32_t (&cb)[4], int t) {
  const int k = t & 15, q = t >> 4;
  uint32_t av[4], ane[4], bv[4], bne[4];
  int as[4], bs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    image_a<MODEL, DT>(ca[u], av[u], as[u], ane[u]);
    image_b<DT>(cb[u], bv[u], bs[u], bne[u]);
  }
  if (MODEL == kAmpere) {
    // poison_stage2 across lanes: the 16 lanes of a group hold k = 0..15 of
    // the same rows (columns); the one at k = 8 takes the inf/NaN code when
    // any of k = 0..7 has it
    const int g = (t & 63) >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t sa = (uint32_t)(__ballot(ane[u] == OP_SPECIAL) >> (16 * g)) & 0xFFu;
      const uint32_t sb = (uint32_t)(__ballot(bne[u] == OP_SPECIAL) >> (16 * g)) & 0xFFu;
      if (k == 8 && sa) ane[u] = OP_SPECIAL;
      if (k == 8 && sb) bne[u] = OP_SPECIAL;
    }
  }
  *(uint4*)&st->a.val[k][4 * q] = make_uint4(av[0], av[1], av[2], av[3]);
  *(int4*)&st->a.sgn[k][4 * q] = make_int4(as[0], as[1], as[2], as[3]);
  *(uint4*)&st->b.val[k][4 * q] = make_uint4(bv[0], bv[1], bv[2], bv[3]);
  *(int4*)&st->b.sgn[k][4 * q] = make_int4(bs[0], bs[1], bs[2], bs[3]);
  // A exponents: rows paired within the lane
  st->a.ne[k >> 1][4 * q + (k & 1)] = ane[0] | ane[1] << 16;
  st->a.ne[k >> 1][4 * q + 2 + (k & 1)] = ane[2] | ane[3] << 16;
  // B exponents: k paired with the adjacent lane
  uint32_t pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = from_lane_xor1(bne[u]);
  if ((k & 1) == 0) {
    *(uint4*)&st->b.ne[k >> 1][4 * q] =
        make_uint4(bne[0] | pb[0] << 16, bne[1] | pb[1] << 16, bne[2] | pb[2] << 16,
                   bne[3] | pb[3] << 16);
  }
  // sign bitmasks: a ballot over the wave gives, for each 16-lane group,
  // the 16 sign bits (k = 0..15) of one row / column
  const int g = (t & 63) >> 4;
  uint32_t am[4], bmk[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    am[u] = (uint32_t)(__ballot(as[u] != 0) >> (16 * g)) & 0xFFFFu;
    bmk[u] = (uint32_t)(__ballot(bs[u] != 0) >> (16 * g)) & 0xFFFFu;
  }
  if (k == 0) {
    if (MODEL == kAmpere) {
      *(uint4*)&st->a.msk[0][4 * q] = make_uint4(am[0] & 0xFF, am[1] & 0xFF, am[2] & 0xFF, am[3] & 0xFF);
      *(uint4*)&st->a.msk[1][4 * q] = make_uint4(am[0] >> 8, am[1] >> 8, am[2] >> 8, am[3] >> 8);
      *(uint4*)&st->b.msk[0][4 * q] = make_uint4(bmk[0] & 0xFF, bmk[1] & 0xFF, bmk[2] & 0xFF, bmk[3] & 0xFF);
      *(uint4*)&st->b.msk[1][4 * q] = make_uint4(bmk[0] >> 8, bmk[1] >> 8, bmk[2] >> 8, bmk[3] >> 8);
    } else {
      *(uint4*)&st->a.msk[0][4 * q] = make_uint4(am[0], am[1], am[2], am[3]);
      *(uint4*)&st->b.msk[0][4 * q] = make_uint4(bmk[0], bmk[1], bmk[2], bmk[3]);
    }
  }
}

// Global loads of step s for lane t (the code of 1.0 outside the matrix).
template <int DT>
__device__ __forceinline__ void fetch(const void* A, const void* B, int64_t M, int64_t N,
                                      int64_t K, int64_t bm, int64_t bn, int64_t s, int t,
                                      uint32_t (&ca)[4], uint32_t (&cb)[4]) {
  const int k = t & 15, q = t >> 4;
  const int64_t kk = 16 * s + k;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t row = bm + 4 * q + u;
    ca[u] = row < M ? load_code<DT>(A, row * K + kk) : PAD_CODE<DT>;
    const int64_t col = bn + 4 * q + u;
    cb[u] = col < N ? load_code<DT>(B, kk * N + col) : PAD_CODE<DT>;
  }
}

// Ampere's stage 1 can cancel exactly with inf/NaN operands in it (say
// inf*0 against 0*NaN: equal codes, equal dummy significands, opposite
// signs), leaving S1 = 0, which stage 2 takes for an empty sum: the step's
// result could then be finite and in range.  So when a row of A (a column
// of B) has an inf/NaN operand among k = 0..7, its code at k = 8 becomes the
// inf/NaN code as well; stage 2 then always holds a term of an inf/NaN
// exponent, the result lands out of range and the step is recomputed
// exactly.  ne: one row's (column's) 16 codes of one step.
__device__ __forceinline__ void poison_stage2(uint32_t (&ne)[16]) {
  bool sp = false;
#pragma unroll
  for (int k = 0; k < 8; ++k) sp |= ne[k] == OP_SPECIAL;
  if (sp) ne[8] = OP_SPECIAL;
}

// Pre-pass: build one operand's images of chain positions [t0, t0 + gridDim.x)
// (workspace layout [block][position - t0][OpImage]), so the GEMM kernel only
// copies them into LDS.  Position p holds K-step step_at(order, p): the
// images are in chain order, whatever the step order.  One 64-lane workgroup
// per (position, block); lane r owns row r of an A block (IS_B false) or
// column r of a B block (IS_B true).
template <int MODEL, int DT, bool IS_B>
__global__ __launch_bounds__(64) void unpack_kernel(const void* __restrict__ src, int64_t limit,
                                                    int64_t K, int64_t N, int64_t t0,
                                                    const int32_t* __restrict__ order,
                                                    uint32_t* __restrict__ ws) {
  const int64_t s = step_at(order, t0 + blockIdx.x, K / 16), blk = blockIdx.y;
  const int r = threadIdx.x;
  const int64_t idx = blk * 64 + r;
  OpImage* img = (OpImage*)(ws + (blk * gridDim.x + blockIdx.x) * IMG_WORDS);
  uint32_t codes[16];
  // an A row segment is 16 consecutive codes: two (or, for E4M3, one)
  // 16-byte loads when the row start is 16-byte aligned
  constexpr int esz = Fmt<DT>::bytes;
  const bool vec = !IS_B && idx < limit &&
                   (((uintptr_t)src | (uintptr_t)(K * esz)) & 15u) == 0;
  if (vec) {
    const uint4* p = (const uint4*)((const char*)src + (idx * K + 16 * s) * esz);
    uint32_t w[8];
    const uint4 v0 = p[0];
    w[0] = v0.x, w[1] = v0.y, w[2] = v0.z, w[3] = v0.w;
    if (esz == 2) {
      const uint4 v1 = p[1];
      w[4] = v1.x, w[5] = v1.y, w[6] = v1.z, w[7] = v1.w;
#pragma unroll
      for (int k = 0; k < 16; ++k) codes[k] = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) codes[k] = (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      codes[k] = PAD_CODE<DT>;
      if (idx < limit)
        codes[k] = IS_B ? load_code<DT>(src, (16 * s + k) * N + idx)
                        : load_code<DT>(src, idx * K + 16 * s + k);
    }
  }
  uint32_t msk = 0, ne[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    uint32_t val;
    int sg;
    if (IS_B) {
      image_b<DT>(codes[k], val, sg, ne[k]);
    } else {
      image_a<MODEL, DT>(codes[k], val, sg, ne[k]);
    }
    img->val[k][r] = val;
    img->sgn[k][r] = sg;
    msk |= (uint32_t)(sg & 1) << k;
  }
  if (MODEL == kAmpere) poison_stage2(ne);
  if (IS_B) {
#pragma unroll
    for (int p = 0; p < 8; ++p) img->ne[p][r] = ne[2 * p] | ne[2 * p + 1] << 16;
  } else {
    // rows (r & ~1, r | 1) share a word; lane r writes k = 2p + (r & 1),
    // taking the other row's code from its partner lane r ^ 1
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t mine = (r & 1) ? ne[2 * p + 1] : ne[2 * p];
      const uint32_t other = from_lane_xor1((r & 1) ? ne[2 * p] : ne[2 * p + 1]);
      img->ne[p][r] = (r & 1) ? (other | mine << 16) : (mine | other << 16);
    }
  }
  if (MODEL == kAmpere) {
    img->msk[0][r] = msk & 0xFFu;
    img->msk[1][r] = msk >> 8;
  } else {
    img->msk[0][r] = msk;
    img->msk[1][r] = 0;
  }
}

// Copy one step's A and B images (2 x 12 KiB) from the workspace into a
// stage with direct global->LDS loads: 24 wave loads of 1 KiB, six per wave.
// w is the wave index, already made wave-uniform, so that every address but
// the lane offset stays in scalar registers.
__device__ __forceinline__ void dma_step(Stage* st, const uint32_t* img_a, const uint32_t* img_b,
                                         int w, int lane) {
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int kb = 6 * w + i;
    const uint32_t* base = kb < 12 ? img_a + kb * 256 : img_b + (kb - 12) * 256;
    __builtin_amdgcn_global_load_lds(
        (const void*)(base + 4 * lane),
        (__attribute__((address_space(3))) void*)((uint32_t*)st + kb * 256), 16, 0, 0);
  }
}

// Words [4*ty + 2*QB, 4*ty + 2*(QB + QN)) of an LDS row: the values of
// the lane's row pairs QB .. QB+QN-1 (or, in the exponent rows of the A
// image, their pair words), placed at their own indices of v.
template <int QB, int QN, typename T>
__device__ __forceinline__ void lds_pairs(const T* row, int ty, T (&v)[4]) {
  static_assert(QN == 2 || (QN == 1 && QB < 2), "one or both row pairs");
  if constexpr (QN == 2) {
    const uint4 x = *(const uint4*)&row[4 * ty];
    v[0] = (T)x.x, v[1] = (T)x.y, v[2] = (T)x.z, v[3] = (T)x.w;
  } else {
    const uint2 x = *(const uint2*)&row[4 * ty + 2 * QB];
    v[2 * QB] = (T)x.x, v[2 * QB + 1] = (T)x.y;
  }
}
template <typename T>
__device__ __forceinline__ void lds_quad(const T* row, int tx, T (&v)[4]) {
  const uint4 x = *(const uint4*)&row[4 * tx];
  v[0] = (T)x.x, v[1] = (T)x.y, v[2] = (T)x.z, v[3] = (T)x.w;
}

// One group of products for the outputs of row pairs QB .. QB+QN-1 of the
// lane's 4x4 tile (rows 2q, 2q+1 form pair q).
//   p0, NP: first k-pair and k-pair count of the group; gmask: sign-mask row.
//   ne_t / X_t: the group's extra term (C, or the Ampere stage-1 sum), its
//   exponent codes paired by output (rows 2q, 2q+1).
// NT_EMPTY: the extra term may be an empty sum (code 0xFFFF, a binary16 NaN
// pattern), which then goes through an integer min.
// STORE_ES keeps every product exponent of pass 1 in registers (2*NP*QN*4
// of them) for pass 2; otherwise pass 2 recomputes them.
// XSH: X_t holds the extra term's one's complement significand XSH bits
// up, with bits below them that are never read (the shifted state form of
// normalise2); its alignment shift is then XSH more, saturating at 31,
// where the arithmetic shift leaves the sign alone, as it should.
// Returns S (signed exact group sum on the grid of the group's emax) and
// mn (= 0x4000 - emax, paired like ne_t) for the pairs it covers.
// INTERLEAVE asks the scheduler to spread pass 2's LDS reads, two per 14
// VALU instructions per row pair (Hopper E4M3 1.6% and BF16 0.6% faster;
// slower for Ampere, which keeps the default schedule).
template <int NP, bool STORE_ES, bool NT_EMPTY, int QB = 0, int QN = 2,
          bool INTERLEAVE = false, int XSH = 0, typename ST>
__device__ __forceinline__ void group(const ST* st, int ty, int tx, int p0, int gmask,
                                      const uint32_t (&ne_t)[2][4], const int (&X_t)[4][4],
                                      int (&S)[4][4], uint32_t (&mn_out)[2][4]) {
  static_assert(STORE_ES || !NT_EMPTY, "an empty extra term needs the stored exponents");
  u16x2 mn[2][4];
  u16x2 es[STORE_ES ? 2 * NP : 1][2][4];
#pragma unroll
  for (int q = QB; q < QB + QN; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) mn[q][c] = as2(ne_t[q][c]);
  // pass 1: exponents of every product and the running maximum per output
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t a[4], b[4];
    lds_pairs<QB, QN>(st->a.ne[p0 + p], ty, a);
    lds_quad(st->b.ne[p0 + p], tx, b);
#pragma unroll
    for (int q = QB; q < QB + QN; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u16x2 e0 = as2(a[2 * q]) + splat_lo(b[c]);
        const u16x2 e1 = as2(a[2 * q + 1]) + splat_hi(b[c]);
        if constexpr (STORE_ES) {
          es[2 * p][q][c] = e0;
          es[2 * p + 1][q][c] = e1;
        }
        if constexpr (!NT_EMPTY) mn[q][c] = min3h(mn[q][c], e0, e1);
      }
  }
  if constexpr (NT_EMPTY) {
#pragma unroll
    for (int q = QB; q < QB + QN; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u16x2 m = __builtin_elementwise_min(mn[q][c], es[0][q][c]);
#pragma unroll
        for (int i = 1; i + 1 < 2 * NP; i += 2) m = min3h(m, es[i][q][c], es[i + 1][q][c]);
        mn[q][c] = __builtin_elementwise_min(m, es[2 * NP - 1][q][c]);
      }
  }
  u16x2 K[2][4];
  int acc[4][4];
#pragma unroll
  for (int q = QB; q < QB + QN; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      K[q][c] = u16x2{SAT, SAT} - mn[q][c];
      // the extra term: one's complement significand shifted onto the grid
      const u16x2 KX = XSH ? u16x2{(unsigned short)(SAT + XSH), (unsigned short)(SAT + XSH)} -
                                 mn[q][c]
                           : K[q][c];
      const uint32_t w = as32(__builtin_elementwise_add_sat(as2(ne_t[q][c]), KX));
      acc[2 * q][c] = X_t[2 * q][c] >> (w & 31);
      acc[2 * q + 1][c] = X_t[2 * q + 1][c] >> ((w >> 16) & 31);
    }
  // pass 2: products, truncating alignment, signed accumulation
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t ane[4] = {0, 0, 0, 0}, bne[4] = {0, 0, 0, 0};
    if constexpr (!STORE_ES) {
      lds_pairs<QB, QN>(st->a.ne[p0 + p], ty, ane);
      lds_quad(st->b.ne[p0 + p], tx, bne);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = 2 * (p0 + p) + j;
      uint32_t a[4];
      int sa[4], b[4], sb[4];
      lds_pairs<QB, QN>(st->a.val[k], ty, a);
      lds_pairs<QB, QN>(st->a.sgn[k], ty, sa);
      lds_quad((const int*)st->b.val[k], tx, b);
      lds_quad(st->b.sgn[k], tx, sb);
#pragma unroll
      for (int q = QB; q < QB + QN; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u16x2 e;
          if constexpr (STORE_ES) {
            e = es[2 * p + j][q][c];
          } else {
            e = as2(ane[2 * q + j]) + (j ? splat_hi(bne[c]) : splat_lo(bne[c]));
          }
          const uint32_t w = as32(__builtin_elementwise_add_sat(e, K[q][c]));
          const int r0 = 2 * q, r1 = 2 * q + 1;
          const int x0 = __mul24(b[c], (int)a[r0]) + sb[c];
          const int x1 = __mul24(b[c], (int)a[r1]) + sb[c];
          const int t0 = x0 >> (w & 31);
          const int t1 = x1 >> ((w >> 16) & 31);
          acc[r0][c] = xad(t0, sa[r0], acc[r0][c]);
          acc[r1][c] = xad(t1, sa[r1], acc[r1][c]);
        }
      if constexpr (INTERLEAVE) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // two LDS reads
          __builtin_amdgcn_sched_group_barrier(0x002, 14 * QN, 0);  // VALU
        }
      }
    }
  }
  // +1 for every negative term: popcount of the XOR of the sign masks, with
  // the extra term's sign in bit 31 (the masks use at most 16 bits)
  uint32_t ma[4], mb[4];
  lds_pairs<QB, QN>(st->a.msk[gmask], ty, ma);
  lds_quad(st->b.msk[gmask], tx, mb);
#pragma unroll
  for (int r = 2 * QB; r < 2 * (QB + QN); ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t nm = (ma[r] ^ mb[c]) | ((uint32_t)X_t[r][c] & 0x80000000u);
      S[r][c] = acc[r][c] + __popc(nm);
    }
#pragma unroll
  for (int q = QB; q < QB + QN; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) mn_out[q][c] = as32(mn[q][c]);
}

// Normalise the group sums of two outputs (one exponent pair): one's
// complement 24-bit significands (shifted by EXTRA onto the next group's
// grid) and their exponent codes L = emax - F + 31 - lz, i.e.
// NE = mn + (F - 31) + lz, by a saturating add so that a zero sum (lz all
// ones) gets 0xFFFF.
// Without an absolute value: U = S + s is |S| ^ s, the one's complement form
// the result takes anyway.  Its signed leading-bit count is |S|'s leading
// zeros lz, and a funnel shift of the pair (U, s) right by 32 - lz gives
// (|S| << lz) ^ s, shifting in copies of the sign.  A second funnel shift of
// (s, that) right by 8 keeps the 24 bits from the leading one down, the
// magnitude cut toward zero, with the sign filled in above them.  A zero
// sum has U = s = 0 and gives 0 whatever lz is.
// XSH = 7 returns the shifted state form instead: the first funnel shift
// alone, by 33 - lz, which puts the leading one at bit 30 and the 24 bits at
// 30 .. 7, with the sign at bit 31 and in everything above; bits 6 .. 0 hold
// bits of |S| ^ s below the cut, which no reader of the form uses (every
// one shifts it right arithmetically by 7 or more).  That needs lz >= 2,
// i.e. |S| < 2^30: an Ampere group sum stays below 2^29.
template <int EXTRA, int F, int XSH = 0>
__device__ __forceinline__ void normalise2(int S0, int S1, uint32_t mn, int& X0, int& X1,
                                           uint32_t& NE) {
  static_assert(XSH == 0 || (XSH == 7 && EXTRA == 0 && F == 23), "shifted form: Ampere only");
  if constexpr (EXTRA != 0) {
    // Hopper's final sum, moved up by EXTRA onto the 25-bit grid: the shift
    // form compiles to v_lshlrev, v_lshrrev and one v_bitop3 per output,
    // as short as the funnel form with its extra bits.
    const int s0 = S0 >> 31, s1 = S1 >> 31;
    const uint32_t m0 = (uint32_t)max(S0, -S0), m1 = (uint32_t)max(S1, -S1);
    const uint32_t lz = ffbh_into_hi(ffbh(m0), m1);
    X0 = (int)(((m0 << (lz & 31)) >> 8) << EXTRA) ^ s0;
    X1 = (int)(((m1 << ((lz >> 16) & 31)) >> 8) << EXTRA) ^ s1;
    const u16x2 base = as2(mn) - u16x2{(unsigned short)(31 - F), (unsigned short)(31 - F)};
    NE = as32(__builtin_elementwise_add_sat(as2(lz), base));
    return;
  }
  const int s0 = S0 >> 31, s1 = S1 >> 31;
  const int U0 = S0 + s0, U1 = S1 + s1;
  // lz = lz0 | lz1 << 16; a funnel shift reads the low 5 bits of its amount
  const uint32_t lz = ffbh_i32_into_hi(ffbh_i32(U0), U1);
  constexpr unsigned short NS = XSH ? 33 : 32;
  const uint32_t nlz = as32(u16x2{NS, NS} - as2(lz));
  const uint32_t W0 = __builtin_amdgcn_alignbit((uint32_t)U0, (uint32_t)s0, nlz);
  const uint32_t W1 = __builtin_amdgcn_alignbit((uint32_t)U1, (uint32_t)s1, nlz >> 16);
  if constexpr (XSH) {
    X0 = (int)W0;
    X1 = (int)W1;
  } else {
    X0 = (int)__builtin_amdgcn_alignbit((uint32_t)s0, W0, 8);
    X1 = (int)__builtin_amdgcn_alignbit((uint32_t)s1, W1, 8);
  }
  const u16x2 base = as2(mn) - u16x2{(unsigned short)(31 - F), (unsigned short)(31 - F)};
  NE = as32(__builtin_elementwise_add_sat(as2(lz), base));
}

// FP32 overflow of a BF16 step (E >= 128, code ne <= NE_OVF), two outputs
// at a time: the state becomes inf, an exponent that dominates every BF16
// product (below 2^256) so that later steps keep it: min(ne, C_INF), i.e.
// E = 1024, or E itself where it is larger already (such a state is a fixed
// point of the step just the same).  Codes above NE_OVF are kept.  Three
// packed operations: t = ne - NE_OVF saturating at 0; x = t * 0xFFFF +
// C_INF clamped, which is C_INF for t = 0 and 0xFFFF otherwise; min(ne, x).
// Only codes the range check lets through (E in [-126, 2047]) are read.
__device__ __forceinline__ uint32_t snap_inf_bf16(uint32_t ne) {
  const u16x2 t = __builtin_elementwise_sub_sat(
      as2(ne), u16x2{(unsigned short)NE_OVF, (unsigned short)NE_OVF});
  uint32_t x;
  asm("v_pk_mad_u16 %0, %1, -1, %2 clamp" : "=v"(x) : "v"(as32(t)), "s"(C_INF | C_INF << 16));
  return as32(__builtin_elementwise_min(as2(ne), as2(x)));
}

// Ampere stage 1 with inf/NaN terms may cancel to S1 = 0, which stage 2
// takes for an empty sum.  Where the stage-1 maximum is an inf/NaN code
// (mn <= SPECIAL_MAX, one half per output), S1 keeps that exponent code, so
// that stage 2 holds a term of an inf/NaN exponent and the step's result
// lands out of range.  For images whose k = 8 code carries the stage-1
// inf/NaN code already (the GEMM's images) this changes nothing.
__device__ __forceinline__ uint32_t keep_special_code(uint32_t mn, uint32_t ne1) {
  const u16x2 sp = __builtin_elementwise_min(
      __builtin_elementwise_sub_sat(as2(mn), u16x2{(unsigned short)SPECIAL_MAX,
                                                   (unsigned short)SPECIAL_MAX}),
      u16x2{1, 1});  // 0: inf/NaN maximum, 1: else
  return as32(as2(mn) + sp * (as2(ne1) - as2(mn)));
}

// One chained MMA step for the lane's 4x4 outputs: state (X, NE) in,
// (Xn, NEn) out.  The lane reads rows 4*ty .. 4*ty+3 of the stage's A image
// and columns 4*tx .. 4*tx+3 of its B image.  A fast result is not
// trustworthy when it is zero, below FP32's normal range or touched by an
// inf/NaN operand: if any output's is not, the whole lane tile is redone
// exactly from the raw codes, redo(r, c, X, ne) returning the new state of
// output (r, c) from its previous state.  (Ampere's stage-1 inf/NaN
// cancellation is caught by the images' k = 8 code, poison_stage2.)
// The Ampere state is carried in normalise2's shifted form (X = the one's
// complement significand << kStateShift, low bits unread): each group sum
// then takes one funnel shift to normalise, and the shift shows up only in
// the extra term's alignment.  redo sees and returns the plain form.
template <int MODEL>
constexpr int kStateShift = MODEL == kAmpere ? 7 : 0;
template <int MODEL, int DT, typename ST, typename REDO>
__device__ __forceinline__ void tile_step(const ST* st, int ty, int tx, const int (&X)[4][4],
                                          const uint32_t (&NE)[2][4], int (&Xn)[4][4],
                                          uint32_t (&NEn)[2][4], REDO&& redo) {
  constexpr int F = Model<MODEL>::F;
  constexpr int XS = kStateShift<MODEL>;
  int S[4][4];
  uint32_t mn[2][4];
  // range check: the largest (NE - NE_OK_LO) mod 2^16 over the 16 outputs
  u16x2 rng = {0, 0};
  // final normalisation, range check and overflow snap of row pair q
  auto finish = [&](int q) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      normalise2<F - 23, F, XS>(S[2 * q][c], S[2 * q + 1][c], mn[q][c], Xn[2 * q][c],
                                Xn[2 * q + 1][c], NEn[q][c]);
      const uint32_t ne = NEn[q][c];
      const u16x2 off = as2(ne) - u16x2{(unsigned short)NE_OK_LO, (unsigned short)NE_OK_LO};
      rng = __builtin_elementwise_max(rng, off);
      // FP32 overflow (L >= 128): the state becomes inf.  FP16 and E4M3
      // products stay below 2^33, so L = 128 already dominates them and a
      // max suffices; BF16 products reach 2^256 and need E >= 1024.
      if (DT == kBF16) {
        NEn[q][c] = snap_inf_bf16(ne);
      } else {
        NEn[q][c] = as32(__builtin_elementwise_max(
            as2(ne), u16x2{(unsigned short)NE_OVF, (unsigned short)NE_OVF}));
      }
    }
  };
  if (MODEL == kAmpere) {
    group<4, true, false, 0, 2, false, XS>(st, ty, tx, 0, 0, NE, X, S, mn);
    int X1[4][4];
    uint32_t NE1[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        normalise2<0, F, XS>(S[2 * q][c], S[2 * q + 1][c], mn[q][c], X1[2 * q][c],
                             X1[2 * q + 1][c], NE1[q][c]);
      }
    group<4, true, true, 0, 2, false, XS>(st, ty, tx, 4, 1, NE1, X1, S, mn);
    finish(0);
    finish(1);
  } else {
    // one row pair at a time: the 16 product exponents of 8 outputs stay in
    // 64 registers
    group<8, true, false, 0, 1, DT != kFP16>(st, ty, tx, 0, 0, NE, X, S, mn);
    finish(0);
    // reload the B operands from LDS for the second pair rather than keep
    // all 16 k-steps of them live across the first
    asm volatile("" ::: "memory");
    group<8, true, false, 1, 1, DT != kFP16>(st, ty, tx, 0, 0, NE, X, S, mn);
    finish(1);
  }
  if ((rng.x > NE_OK_SPAN) | (rng.y > NE_OK_SPAN)) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // recompute the whole 4x4 tile from the previous state
        const uint2 v0 = redo(2 * q, c, X[2 * q][c] >> XS, NE[q][c] & 0xFFFFu);
        const uint2 v1 = redo(2 * q + 1, c, X[2 * q + 1][c] >> XS, NE[q][c] >> 16);
        Xn[2 * q][c] = (int)(v0.x << XS);
        Xn[2 * q + 1][c] = (int)(v1.x << XS);
        NEn[q][c] = v0.y | v1.y << 16;
      }
  }
}

// Waves per SIMD the register allocation is sized for.  A step keeps 64
// product exponents in registers (an Ampere group over the whole tile, a
// Hopper group over half of it) and fits three; its only spills sit around
// the rare recompute calls.  The in-kernel image build needs more registers
// and stays at two.
template <int MODEL, bool DMA>
constexpr int kWavesPerSimd = DMA ? 3 : 2;

// DMA = true: the operand images come from the pre-pass workspace (ws_a,
// ws_b, holding steps [i0, i0 + istride) of every block) by direct
// global->LDS copies; DMA = false: the kernel builds them from the raw codes
// (no workspace).  The kernel chains the ns steps that start at step s0 (all
// K/16 of them for a plain GEMM; one run of a split-K schedule, or one chunk
// of steps when the workspace holds fewer than all of them, otherwise).
// With gridDim.z > 1 the z-th slice of the grid chains the ns steps that
// start at s0 + z*ns instead, from +0 when z > 0, and stores into the D of
// out moved on by z*zstride words: the runs of a split-K schedule side by
// side.  Steps are chain positions: position p applies K-step
// step_at(order, p) (p itself when order is NULL); the workspace images are
// already in position order.  The K loop is unrolled twice so that the accumulator state
// alternates between two register sets instead of being copied back every
// step.
template <int MODEL, int DT, bool DMA>
__global__ __launch_bounds__(NT, (kWavesPerSimd<MODEL, DMA>)) void gemm_fast_kernel(
    const void* __restrict__ A, const void* __restrict__ B, const uint32_t* C0, Sink out0,
    int64_t M, int64_t N, int64_t K, int64_t s00, int64_t ns,
    const uint32_t* __restrict__ ws_a, const uint32_t* __restrict__ ws_b, int64_t i0,
    int64_t istride, int64_t zstride, const int32_t* __restrict__ order) {
  // the two stages of the double buffer are two LDS variables, not one
  // array: the compiler can then tell that the copy into one (a
  // global->LDS load, counted in vmcnt) cannot alias the reads of the
  // other, and does not wait for the copy before the step that overlaps it
  __shared__ Stage stage0, stage1;
  const int64_t z = blockIdx.z;
  const uint32_t* const C = z ? nullptr : C0;
  const int64_t s0 = s00 + z * ns;
  Sink out = out0;
  if (out.D) out.D += z * zstride;
  const int t = threadIdx.x;
  const int ty = t >> 4, tx = t & 15;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int64_t bm = (int64_t)blockIdx.y * BM, bn = (int64_t)blockIdx.x * BN;
  const int64_t nsteps = ns;  // steps chained here

  int X[4][4], Xn[4][4];
  uint32_t NE[2][4], NEn[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t ne[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t row = bm + 4 * ty + 2 * q + h, col = bn + 4 * tx + c;
        const uint32_t cbits = (C && row < M && col < N) ? C[row * N + col] : 0u;
        bits_to_state<MODEL>(cbits, X[2 * q + h][c], ne[h]);
        X[2 * q + h][c] = (int)((uint32_t)X[2 * q + h][c] << kStateShift<MODEL>);
      }
      NE[q][c] = ne[0] | ne[1] << 16;
    }

  const uint32_t* img_a =
      DMA ? ws_a + ((int64_t)blockIdx.y * istride + (s0 - i0)) * IMG_WORDS : nullptr;
  const uint32_t* img_b =
      DMA ? ws_b + ((int64_t)blockIdx.x * istride + (s0 - i0)) * IMG_WORDS : nullptr;
  uint32_t ca[4], cb[4];
  // fill of stage s (local step s, absolute step s0 + s): start it (before
  // the previous step's compute), end it
  auto begin_fill = [&](Stage* st, int64_t s) {
    if constexpr (DMA) {
      dma_step(st, img_a + s * IMG_WORDS, img_b + s * IMG_WORDS, w, lane);
    } else {
      fetch<DT>(A, B, M, N, K, bm, bn, step_at(order, s0 + s, K / 16), t, ca, cb);
    }
  };
  auto end_fill = [&](Stage* st) {
    if constexpr (DMA) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      produce<MODEL, DT>(st, ca, cb, t);
    }
  };
  if (nsteps > 0) {
    begin_fill(&stage0, 0);
    end_fill(&stage0);
  }
  __syncthreads();

  // the exact recompute of output (r, c) of the lane's tile at step ks
  auto redo_at = [&](int64_t ks) {
    return [=](int r, int c, int x, uint32_t ne) {
      return slow_step<MODEL, DT>(A, B, M, N, K, order, ks, r, c, x, ne);
    };
  };
  for (int64_t s = 0; s < nsteps; s += 2) {
    step_priority(s);
    if (s + 1 < nsteps) begin_fill(&stage1, s + 1);
    tile_step<MODEL, DT>(&stage0, ty, tx, X, NE, Xn, NEn, redo_at(s0 + s));
    if (s + 1 < nsteps) end_fill(&stage1);
    __syncthreads();
    if (s + 1 >= nsteps) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) X[r][c] = Xn[r][c];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) NE[q][c] = NEn[q][c];
      break;
    }
    step_priority(s + 1);
    if (s + 2 < nsteps) begin_fill(&stage0, s + 2);
    tile_step<MODEL, DT>(&stage1, ty, tx, Xn, NEn, X, NE, redo_at(s0 + s + 1));
    if (s + 2 < nsteps) end_fill(&stage0);
    __syncthreads();
  }

  // the epilogue's addresses are recomputed from opaque copies of the lane
  // indices, so that the compiler does not keep the prologue's 64-bit
  // addresses live (spilled) across the K loop
  int ety = ty, etx = tx;
  asm volatile("" : "+v"(ety), "+v"(etx));
  const int64_t ebm = (int64_t)blockIdx.y * BM, ebn = (int64_t)blockIdx.x * BN;
  uint32_t rowx[4] = {0, 0, 0, 0};
  uint32_t nbad = 0;
  unsigned long long first = ~0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t row = ebm + 4 * ety + r, col = ebn + 4 * etx + c;
      const uint32_t d = state_to_bits<MODEL>(X[r][c] >> kStateShift<MODEL>,
                                              half16(NE[r >> 1][c], r & 1));
      if (row < M && col < N) {
        const int64_t idx = row * N + col;
        if (out.claimed) {
          const uint32_t x = d ^ out.claimed[idx];
          rowx[r] ^= x;
          if (x) {
            ++nbad;
            first = (unsigned long long)idx < first ? (unsigned long long)idx : first;
          }
        } else {
          const uint32_t v = out.accumulate ? fp32_add_rne(out.D[idx], d) : d;
          out.D[idx] = v;
          rowx[r] ^= v;
        }
      }
    }
  if (out.claimed) report_mismatches(out.report, nbad, first);
  uint32_t* const xorsum = out.xorsum;
  if (xorsum) {
    // XOR across the 16 lanes that share these rows (one 16-lane row of the wave)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t v = rowx[r];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) v ^= __shfl_xor(v, off, 16);
      const int64_t row = ebm + 4 * ety + r;
      if (etx == 0 && row < M && v) atomicXor(&xorsum[row], v);
    }
  }
}

// The ordered reduction of split-K partial results P[0..runs) (each M x N):
// D = ((P0 + P1) + P2) ... in FP32 round-to-nearest-even, one lane per
// output, and the per-row XOR of the final D.
__global__ __launch_bounds__(256) void reduce_runs_kernel(const uint32_t* __restrict__ P,
                                                         int64_t runs, int64_t M, int64_t N,
                                                         uint32_t* __restrict__ D,
                                                         uint32_t* __restrict__ xorsum) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    uint32_t v = 0;
    if (col < N) {
      const int64_t idx = row * N + col;
      v = P[idx];
      for (int64_t r = 1; r < runs; ++r) v = fp32_add_rne(v, P[r * M * N + idx]);
      D[idx] = v;
    }
    if (xorsum) {
      const uint32_t w = wave_xor(v);
      if ((threadIdx.x & 63) == 0 && w) atomicXor(&xorsum[row], w);
    }
  }
}

}  // namespace fastk

// Shapes the tiled kernel takes: the GEMM grid is (N blocks, M blocks) and
// the pre-pass grids are (K/16, M blocks) and (K/16, N blocks), so both
// block counts must fit gridDim.y (65535) and K/16 gridDim.x.
inline bool gemm_fast_supported(int64_t M, int64_t N, int64_t K) {
  return M > 0 && N > 0 && K >= 16 && (M + fastk::BM - 1) / fastk::BM <= 65535 &&
         (N + fastk::BN - 1) / fastk::BN <= 65535 && K / 16 <= INT32_MAX;
}

// Bytes of pre-pass workspace for an M x N x K GEMM (operand images).
inline int64_t gemm_fast_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t mb = (M + fastk::BM - 1) / fastk::BM, nb = (N + fastk::BN - 1) / fastk::BN;
  return (mb + nb) * (K / 16) * (int64_t)sizeof(fastk::OpImage);
}

// order: NULL for the forward order, else the K-step of each chain position
// (step_at); every schedule below works on chain positions.
// ws: NULL for the in-kernel image build, else a workspace that holds the
// images of ws_steps steps of every A block and every B block
// (gemm_fast_workspace_bytes(M, N, 16 * ws_steps) bytes).
// splits > 1 (a divisor of K/16): the split-K schedule.  Run r chains steps
// [r*T/splits, (r+1)*T/splits) of the T = K/16 steps, from C for r = 0 and
// from +0 otherwise, giving P_r, and D = ((P0 + P1) + P2) ... in FP32
// round-to-nearest-even (fp32_add_rne).  With a partials buffer of
// splits x M x N words and images of all T steps, the runs are computed side
// by side into it and then added in run order (reduce_runs_kernel, which
// also takes the xorsum); otherwise the runs are launched in order and each
// later one adds its partial result into D, the last one taking the xorsum.
// A workspace too small for all T steps is filled once per run, or, when it
// cannot hold a whole run, run 0 of an emulating call is cut into chunks of
// ws_steps steps, each restarting from the D that the previous chunk wrote:
// every step's result is an FP32 value, so the chain through D is the same
// chain.  What remains (a later run, the audit compare) builds its images in
// LDS.
template <int MODEL, int DT>
inline void gemm_fast_launch(const void* A, const void* B, const uint32_t* C, const Sink& out,
                             int64_t M, int64_t N, int64_t K, void* ws, int64_t ws_steps,
                             hipStream_t s, int64_t splits = 1, uint32_t* partials = nullptr,
                             const int32_t* order = nullptr) {
  const int64_t mb = (M + fastk::BM - 1) / fastk::BM, nb = (N + fastk::BN - 1) / fastk::BN;
  const int64_t nsteps = K / 16, per = nsteps / splits;
  const dim3 grid((unsigned)nb, (unsigned)mb);
  if (!ws) ws_steps = 0;
  uint32_t* ws_a = (uint32_t*)ws;
  uint32_t* ws_b = ws ? ws_a + mb * ws_steps * fastk::IMG_WORDS : nullptr;
  // the images of steps [t0, t0 + n), n <= ws_steps
  auto prepass = [&](int64_t t0, int64_t n) {
    fastk::unpack_kernel<MODEL, DT, false>
        <<<dim3((unsigned)n, (unsigned)mb), dim3(64), 0, s>>>(A, M, K, N, t0, order, ws_a);
    fastk::unpack_kernel<MODEL, DT, true>
        <<<dim3((unsigned)n, (unsigned)nb), dim3(64), 0, s>>>(B, N, K, N, t0, order, ws_b);
  };
  // steps [t0, t0 + n) from c into o, with the images of steps [i0, i0 + istride)
  // in the workspace (istride = 0: built in LDS)
  auto chain = [&](const uint32_t* c, const Sink& o, int64_t t0, int64_t n, int64_t i0,
                   int64_t istride) {
    if (istride > 0) {
      fastk::gemm_fast_kernel<MODEL, DT, true><<<grid, dim3(fastk::NT), 0, s>>>(
          A, B, c, o, M, N, K, t0, n, ws_a, ws_b, i0, istride, 0, order);
    } else {
      fastk::gemm_fast_kernel<MODEL, DT, false><<<grid, dim3(fastk::NT), 0, s>>>(
          A, B, c, o, M, N, K, t0, n, nullptr, nullptr, 0, 0, 0, order);
    }
  };
  const bool whole = ws_steps >= nsteps;
  if (whole) prepass(0, nsteps);
  if (whole && partials && splits > 1) {
    // every run at once, each into its own M x N partial result, then the
    // ordered reduction (and the xorsum of the final D)
    Sink o = out;
    o.D = partials;
    o.xorsum = nullptr;
    o.accumulate = 0;
    fastk::gemm_fast_kernel<MODEL, DT, true>
        <<<dim3((unsigned)nb, (unsigned)mb, (unsigned)splits), dim3(fastk::NT), 0, s>>>(
            A, B, C, o, M, N, K, 0, per, ws_a, ws_b, 0, nsteps, M * N, order);
    const int64_t rows = M < 32768 ? M : 32768;
    fastk::reduce_runs_kernel<<<dim3((unsigned)((N + 255) / 256), (unsigned)rows), dim3(256),
                                0, s>>>(partials, splits, M, N, out.D, out.xorsum);
    return;
  }
  for (int64_t r = 0; r < splits; ++r) {
    Sink o = out;
    o.accumulate = r > 0;
    if (r + 1 < splits) o.xorsum = nullptr;
    const uint32_t* c = r == 0 ? C : nullptr;
    const int64_t t0 = r * per;
    if (whole) {
      chain(c, o, t0, per, 0, nsteps);
    } else if (ws_steps >= per) {
      prepass(t0, per);
      chain(c, o, t0, per, t0, per);
    } else if (r > 0 || !out.D || ws_steps == 0) {
      chain(c, o, t0, per, 0, 0);
    } else {
      for (int64_t u = 0; u < per; u += ws_steps) {
        const int64_t n = per - u < ws_steps ? per - u : ws_steps;
        Sink oc = o;
        if (u + n < per) oc.xorsum = nullptr;
        prepass(t0 + u, n);
        chain(u == 0 ? c : out.D, oc, t0 + u, n, t0 + u, n);
      }
    }
  }
}

}  // namespace mmaemu
