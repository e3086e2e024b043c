// tiles_fast.h -- independent 16x16x16 MMA steps (mma_emulate_tiles) with
// the tiled GEMM kernel's own step (gemm_fast.h: group, normalise2,
// tile_step).  One 64-lane wave takes four tiles at a time:
//
//  * the four tiles' A rows and B columns fill one GEMM stage, A rows and
//    B columns 16u .. 16u+15 belonging to tile u; the wave builds it from
//    the raw codes with the GEMM's in-kernel image builder (produce), eight
//    operands per lane and call;
//  * lane (u, a, b) owns rows 4a .. 4a+3 and columns 4b .. 4b+3 of tile u,
//    which is the GEMM lane tile (ty, tx) = (4u + a, 4u + b): its 16
//    outputs share every operand read from LDS four times over, and their
//    exponent codes pair by output row as in the GEMM;
//  * C is decoded into the accumulator state, one chained step is taken,
//    and D and the per-tile XOR are written.  A result that is zero,
//    FP32-subnormal or touched by inf/NaN is redone by step_generic from the
//    tile's raw codes and C, one output at a time: each lane walks its own
//    such outputs, so a wave pays for the largest count on one lane, not
//    for every output slot that any lane needs;
//  * the next four tiles' codes and the lane's C words are loaded while the
//    current ones are computed (grid-stride loop).
#pragma once

#include "gemm_fast.h"

namespace mmaemu {
namespace tilek {

using namespace fastk;

constexpr int TPW = 4;  // tiles per wave

// A GEMM stage without the padding of the 12 KiB images (those exist only
// for whole-image copies): 22,848 bytes, seven waves per CU.  Declared
// 16-byte aligned so that the image builder's 16-byte stores stay single
// b128 writes (at 4-byte alignment each became two two-word writes, whose
// lanes at k and k + 8 collide on the same LDS banks).
struct alignas(16) TileImage {
  uint32_t val[16][PAD];
  int32_t sgn[16][PAD];
  uint32_t ne[8][PAD];
  uint32_t msk[2][PAD];
};
struct TileStage {
  TileImage a, b;
};

// The exact step of output (row, col) of a live tile, from its raw codes
// and C (read before this output's D is written, so C may be D).
template <int MODEL, int DT>
__device__ __noinline__ uint32_t redo_output(const void* A, const void* B, const uint32_t* C,
                                             int64_t tile, int row, int col) {
  uint32_t a[16], b[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    a[k] = load_code<DT>(A, tile * 256 + 16 * row + k);
    b[k] = load_code<DT>(B, tile * 256 + 16 * k + col);
  }
  return step_generic<MODEL, DT>(C ? C[tile * 256 + 16 * row + col] : 0u, a, b);
}

template <int MODEL, int DT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void tiles_fast_kernel(
    const void* __restrict__ A, const void* __restrict__ B,
    const uint32_t* C,  // may equal D
    uint32_t* D, uint32_t* __restrict__ xorsum, int64_t ntiles) {
  __shared__ TileStage st;
  const int lane = threadIdx.x;
  // staging role: k = lane & 15; A rows and B columns 4q .. 4q+3 of each tile
  const int k = lane & 15, q = lane >> 4;
  // output role: tile u of the four, rows 4a.., columns 4b..
  const int u = lane >> 4, a = (lane >> 2) & 3, b = lane & 3;
  const int64_t ngroups = (ntiles + TPW - 1) / TPW;
  const bool vec = (((uintptr_t)C | (uintptr_t)D) & 15u) == 0;

  uint32_t ca[TPW][4], cb[TPW][4], cbits[4][4];
  // the codes of tiles TPW*g .. TPW*g + TPW-1 for the staging role and the
  // C words of the lane's outputs; a full group loads from one base per
  // operand at constant offsets, the last (partial) group reads zero codes
  // past the end
  auto load = [&](int64_t g) {
    const int64_t t0 = TPW * g;
    const int64_t ia = t0 * 256 + 64 * q + k, ib = t0 * 256 + 16 * k + 4 * q;
    const int64_t ic = (t0 + u) * 256 + 64 * a + 4 * b;
    if (t0 + TPW <= ntiles) {
#pragma unroll
      for (int v = 0; v < TPW; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ca[v][w] = load_code<DT>(A, ia + 256 * v + 16 * w);
          cb[v][w] = load_code<DT>(B, ib + 256 * v + w);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (C && vec) {
          const uint4 x = *(const uint4*)(C + ic + 16 * r);
          cbits[r][0] = x.x, cbits[r][1] = x.y, cbits[r][2] = x.z, cbits[r][3] = x.w;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) cbits[r][c] = C ? C[ic + 16 * r + c] : 0u;
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < TPW; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ca[v][w] = t0 + v < ntiles ? load_code<DT>(A, ia + 256 * v + 16 * w) : 0u;
          cb[v][w] = t0 + v < ntiles ? load_code<DT>(B, ib + 256 * v + w) : 0u;
        }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          cbits[r][c] = (C && t0 + u < ntiles) ? C[ic + 16 * r + c] : 0u;
    }
  };
  int64_t g = blockIdx.x;
  if (g < ngroups) load(g);
  for (; g < ngroups; g += gridDim.x) {
    __syncthreads();  // the previous tiles' LDS reads are done
    // an opaque copy of the lane index, so that the compiler recomputes the
    // staging addresses here instead of keeping them live (spilled) across
    // the loop
    int sl = lane;
    asm volatile("" : "+v"(sl));
#pragma unroll
    for (int v = 0; v < TPW; ++v) produce<MODEL, DT>(&st, ca[v], cb[v], sl + 64 * v);
    __syncthreads();

    const int64_t tile = TPW * g + u;
    const bool live = tile < ntiles;
    // output (4a + r, 4b + c) of the tile sits at base + 16 r + c
    const int64_t base = tile * 256 + 64 * a + 4 * b;
    int X[4][4], Xn[4][4];
    uint32_t NE[2][4], NEn[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t ne[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) bits_to_state<MODEL>(cbits[2 * p + h][c], X[2 * p + h][c], ne[h]);
        NE[p][c] = ne[0] | ne[1] << 16;
      }
    if (g + gridDim.x < ngroups) load(g + gridDim.x);
    uint32_t bad = 0;
    tile_step<MODEL, DT, true>(&st, 4 * u + a, 4 * u + b, X, NE, Xn, NEn,
                               [](int, int, int, uint32_t) { return make_uint2(0, 0); }, &bad);
    if (!live) bad = 0;
    // the fast results: every output not flagged in bad
    uint32_t xs = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        d[c] = state_to_bits<MODEL>(Xn[r][c], half16(NEn[r >> 1][c], r & 1));
        xs ^= (bad >> (4 * r + c)) & 1u ? 0u : d[c];
      }
      if (live) {
        if (vec && ((bad >> (4 * r)) & 15u) == 0) {
          *(uint4*)(D + base + 16 * r) = make_uint4(d[0], d[1], d[2], d[3]);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (!((bad >> (4 * r + c)) & 1u)) D[base + 16 * r + c] = d[c];
        }
      }
    }
    // the flagged ones, exactly, one per lane at a time
    for (uint32_t m = bad; m; m &= m - 1) {
      const int i = __builtin_ctz(m);
      const int r = i >> 2, c = i & 3;
      const uint32_t d = redo_output<MODEL, DT>(A, B, C, tile, 4 * a + r, 4 * b + c);
      D[base + 16 * r + c] = d;
      xs ^= d;
    }
    if (xorsum) {
      // the tile's 256 words: XOR over the 16 lanes of tile u
      xs = row16_xor(xs);
      if ((lane & 15) == 0 && live) xorsum[tile] = xs;
    }
  }
}

}  // namespace tilek
}  // namespace mmaemu
