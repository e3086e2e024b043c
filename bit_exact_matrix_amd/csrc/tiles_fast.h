// tiles_fast.h -- independent 16x16x16 MMA steps (mma_emulate_tiles), one
// workgroup per tile and one lane per output, with the arithmetic of the
// tiled GEMM kernel (gemm_fast.h) applied to a single output:
//
//  * the workgroup decodes the tile's 512 operands once into LDS (two per
//    lane): A significands pre-shifted onto the group grid and B's signed,
//    0/-1 sign masks, 16-bit exponent codes paired over consecutive k, and
//    per-row / per-column sign bitmasks; B is stored transposed so that
//    every lane reads both of its operand rows contiguously over k;
//  * each lane forms the exponents of two products per packed add, keeps
//    the group maximum with packed binary16 minimum3, gets both alignment
//    distances from one saturating packed add, and accumulates each product
//    with v_mad_i32_i24 (one's complement in B's sign), an arithmetic shift
//    (magnitude truncation) and v_xad_u32 (A's sign), plus one popcount per
//    group for the negative terms;
//  * a result that is zero, below FP32's normal range or touched by inf/NaN
//    is recomputed by step_generic from the tile's raw codes.
#pragma once

#include "gemm_fast.h"

namespace mmaemu {
namespace tilek {

using namespace fastk;

constexpr int RP = 20;  // LDS row pitch in words: 16-byte aligned, conflict-free b128 rows
constexpr int EP = 12;  // the same for the 8-word rows of exponent-code pairs

// One group of the lane's output: products k in [2*p0, 2*(p0+NP)), the extra
// term (X_t, ne_t).  e holds the pass-1 exponent pairs for pass 2.
template <int NP, bool NT_EMPTY>
__device__ __forceinline__ int group1(const uint32_t (&av)[16], const int (&as)[16],
                                      const int (&bv)[16], const int (&bs)[16],
                                      const uint32_t (&ae)[8], const uint32_t (&be)[8], int p0,
                                      uint32_t ne_t, int X_t, uint32_t gmask, uint32_t& mn_out) {
  u16x2 e[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) e[p] = as2(ae[p0 + p]) + as2(be[p0 + p]);
  u16x2 m = splat_lo(ne_t);
  int p = 0;
  if constexpr (NT_EMPTY) {  // the code 0xFFFF (empty sum) is a binary16 NaN pattern
    m = __builtin_elementwise_min(m, e[0]);
    p = 1;
  }
  for (; p + 1 < NP; p += 2) m = min3h(m, e[p], e[p + 1]);
  if (p < NP) m = min3h(m, e[p], e[p]);
  m = __builtin_elementwise_min(m, u16x2{m.y, m.x});  // both halves: the group minimum
  const u16x2 K = u16x2{SAT, SAT} - m;
  const uint32_t wt = as32(__builtin_elementwise_add_sat(splat_lo(ne_t), K));
  int acc = X_t >> (wt & 31);
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const uint32_t w = as32(__builtin_elementwise_add_sat(e[q], K));
    const int k0 = 2 * (p0 + q), k1 = k0 + 1;
    const int x0 = __mul24(bv[k0], (int)av[k0]) + bs[k0];
    const int x1 = __mul24(bv[k1], (int)av[k1]) + bs[k1];
    acc = xad(x0 >> (w & 31), as[k0], acc);
    acc = xad(x1 >> ((w >> 16) & 31), as[k1], acc);
  }
  mn_out = as32(m) & 0xFFFFu;
  return acc + __popc(gmask | ((uint32_t)X_t & 0x80000000u));
}

// Normalise one group sum: one's complement significand (shifted by EXTRA
// onto the next grid) and its exponent code, 0xFFFF for a zero sum.
template <int EXTRA, int F>
__device__ __forceinline__ void normalise1(int S, uint32_t mn, int& X, uint32_t& NE) {
  const int s = S >> 31;
  const uint32_t m = (uint32_t)max(S, -S);
  const uint32_t lz = ffbh(m);
  X = (int)(((m << (lz & 31)) >> 8) << EXTRA) ^ s;
  const u16x2 base = splat_lo(mn) - u16x2{(unsigned short)(31 - F), (unsigned short)(31 - F)};
  NE = as32(__builtin_elementwise_add_sat(splat_lo(lz), base)) & 0xFFFFu;
}

template <int MODEL, int DT>
__global__ __launch_bounds__(256) void tiles_fast_kernel(const void* __restrict__ A,
                                                         const void* __restrict__ B,
                                                         const uint32_t* C,  // may equal D
                                                         uint32_t* D,
                                                         uint32_t* __restrict__ xorsum,
                                                         int64_t ntiles) {
  constexpr int F = Model<MODEL>::F;
  __shared__ uint32_t s_av[16][RP], s_bv[16][RP];  // [row i][k], [column j][k]
  __shared__ int s_as[16][RP], s_bs[16][RP];
  __shared__ uint32_t s_ae[16][EP], s_be[16][EP];  // exponent codes of k = 2p, 2p+1
  __shared__ uint32_t s_am[16], s_bm[4][16];       // sign bitmasks over k
  __shared__ uint32_t s_wx[4];
  const int tid = threadIdx.x, i = tid >> 4, j = tid & 15, wv = tid >> 6;

  // grid-stride loop over tiles; the next tile's codes are loaded while the
  // current one is computed.  Lane (i, j) loads A[i][j] (row i, k = j),
  // B[i][j] (k = i, column j) and C[i][j].
  int64_t tile = blockIdx.x;
  uint32_t ca = 0, cb = 0, cc = 0;
  if (tile < ntiles) {
    ca = load_code<DT>(A, tile * 256 + tid);
    cb = load_code<DT>(B, tile * 256 + tid);
    cc = C ? C[tile * 256 + tid] : 0u;
  }
  for (; tile < ntiles; tile += gridDim.x) {
    const int64_t base = tile * 256;
    const uint32_t code_a = ca, code_b = cb, cbits = cc;
    const int64_t next = tile + gridDim.x;
    if (next < ntiles) {
      ca = load_code<DT>(A, next * 256 + tid);
      cb = load_code<DT>(B, next * 256 + tid);
      cc = C ? C[next * 256 + tid] : 0u;
    }
    __syncthreads();  // the previous tile's LDS reads are done
    {
      uint32_t v, ne;
      int s;
      image_a<MODEL, DT>(code_a, v, s, ne);
      s_av[i][j] = v;
      s_as[i][j] = s;
      const uint32_t ne_a1 = __shfl_xor(ne, 1, 64);  // the same row's code at k ^ 1
      if ((j & 1) == 0) s_ae[i][j >> 1] = ne | ne_a1 << 16;
      const uint64_t bal_a = __ballot(s != 0);       // bit 16*(i&3) + k: row i's signs
      if (j == 0) s_am[i] = (uint32_t)(bal_a >> (16 * (i & 3))) & 0xFFFFu;

      image_b<DT>(code_b, v, s, ne);
      s_bv[j][i] = (uint32_t)v;
      s_bs[j][i] = s;
      const uint32_t ne_b1 = __shfl_xor(ne, 16, 64);  // the same column's code at k ^ 1
      if ((i & 1) == 0) s_be[j][i >> 1] = ne | ne_b1 << 16;
      // column j's signs at k = 4*wv + r sit in bits 16*r + j of this wave's ballot
      const uint64_t bal_b = __ballot(s != 0);
      if ((i & 3) == 0) {
        uint32_t c4 = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) c4 |= (uint32_t)((bal_b >> (16 * r + j)) & 1u) << r;
        s_bm[wv][j] = c4 << (4 * wv);
      }
    }
    __syncthreads();

    uint32_t av[16], ae[8], be[8];
    int as[16], bv[16], bs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 a4 = *(const uint4*)&s_av[i][4 * q];
      const int4 sa4 = *(const int4*)&s_as[i][4 * q];
      const int4 b4 = *(const int4*)&s_bv[j][4 * q];
      const int4 sb4 = *(const int4*)&s_bs[j][4 * q];
      av[4 * q] = a4.x, av[4 * q + 1] = a4.y, av[4 * q + 2] = a4.z, av[4 * q + 3] = a4.w;
      as[4 * q] = sa4.x, as[4 * q + 1] = sa4.y, as[4 * q + 2] = sa4.z, as[4 * q + 3] = sa4.w;
      bv[4 * q] = b4.x, bv[4 * q + 1] = b4.y, bv[4 * q + 2] = b4.z, bv[4 * q + 3] = b4.w;
      bs[4 * q] = sb4.x, bs[4 * q + 1] = sb4.y, bs[4 * q + 2] = sb4.z, bs[4 * q + 3] = sb4.w;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 x = *(const uint4*)&s_ae[i][4 * q];
      const uint4 y = *(const uint4*)&s_be[j][4 * q];
      ae[4 * q] = x.x, ae[4 * q + 1] = x.y, ae[4 * q + 2] = x.z, ae[4 * q + 3] = x.w;
      be[4 * q] = y.x, be[4 * q + 1] = y.y, be[4 * q + 2] = y.z, be[4 * q + 3] = y.w;
    }
    const uint32_t neg = s_am[i] ^ (s_bm[0][j] | s_bm[1][j] | s_bm[2][j] | s_bm[3][j]);

    int Xc;
    uint32_t nec;
    bits_to_state<MODEL>(cbits, Xc, nec);
    int X;
    uint32_t NE, mn;
    if (MODEL == kAmpere) {
      const int S1 = group1<4, false>(av, as, bv, bs, ae, be, 0, nec, Xc, neg & 0xFFu, mn);
      int X1;
      uint32_t NE1;
      normalise1<0, F>(S1, mn, X1, NE1);
      const int S = group1<4, true>(av, as, bv, bs, ae, be, 4, NE1, X1, neg >> 8, mn);
      normalise1<F - 23, F>(S, mn, X, NE);
    } else {
      const int S = group1<8, false>(av, as, bv, bs, ae, be, 0, nec, Xc, neg, mn);
      normalise1<F - 23, F>(S, mn, X, NE);
    }
    uint32_t d;
    if ((unsigned short)(NE - NE_OK_LO) > NE_OK_SPAN) {
      // zero, FP32-subnormal, inf/NaN: the exact per-output step
      uint32_t a[16], b[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        a[k] = load_code<DT>(A, base + 16 * i + k);
        b[k] = load_code<DT>(B, base + 16 * k + j);
      }
      d = step_generic<MODEL, DT>(cbits, a, b);
    } else {
      d = state_to_bits<MODEL>(X, NE);  // L >= 128 (FP32 overflow) gives the signed inf
    }
    D[base + tid] = d;
    if (xorsum) {
      const uint32_t w = wave_xor(d);
      if ((tid & 63) == 0) s_wx[wv] = w;
      __syncthreads();
      if (tid == 0) xorsum[tile] = s_wx[0] ^ s_wx[1] ^ s_wx[2] ^ s_wx[3];
    }
  }
}

}  // namespace tilek
}  // namespace mmaemu
