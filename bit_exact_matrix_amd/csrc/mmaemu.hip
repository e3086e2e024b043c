// mmaemu.hip -- libmmaemu.so: kernels and C ABI of the MI355X bit-exact
// tile-MMA emulator.  The interface and the arithmetic it implements are
// documented in include/mmaemu.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/mmaemu.h"
#include "mmaemu_common.h"
#include "gemm_fast.h"
#include "gemm_narrow.h"
#include "tiles_fast.h"

using namespace mmaemu;

namespace {

constexpr int kSpecVersion = 1;

// --------------------------------------------------- reference GEMM path
// One lane per output, the chained steps read straight from global memory.
// Kept as the simple, fully general path (any shape, any input bits).  It
// chains the ns steps that start at step s0.
template <int MODEL, int DT>
__global__ __launch_bounds__(256) void gemm_reference_kernel(
    const void* __restrict__ A, const void* __restrict__ B, const uint32_t* C, Sink out,
    int64_t M, int64_t N, int64_t K, int64_t s0, int64_t ns) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = col < N;
  uint32_t nbad = 0;
  unsigned long long first = ~0ull;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    uint32_t c = 0, x = 0;
    if (live) {
      c = C ? C[row * N + col] : 0u;
      for (int64_t t = s0; t < s0 + ns; ++t) {
        uint32_t a[16], b[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          a[k] = load_code<DT>(A, row * K + 16 * t + k);
          b[k] = load_code<DT>(B, (16 * t + k) * N + col);
        }
        c = step_generic<MODEL, DT>(c, a, b);
      }
      const int64_t idx = row * N + col;
      if (out.claimed) {
        x = c ^ out.claimed[idx];
        if (x) {
          ++nbad;
          first = (unsigned long long)idx < first ? (unsigned long long)idx : first;
        }
      } else {
        x = out.accumulate ? fp32_add_rne(out.D[idx], c) : c;
        out.D[idx] = x;
      }
    }
    if (out.xorsum) {
      const uint32_t w = wave_xor(x);
      if ((threadIdx.x & 63) == 0 && w) atomicXor(&out.xorsum[row], w);
    }
  }
  if (out.claimed) report_mismatches(out.report, nbad, first);
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// report = {0 mismatches, no mismatching index}
__global__ void init_report_kernel(unsigned long long* report) {
  if (threadIdx.x == 0) {
    report[0] = 0ull;
    report[1] = ~0ull;
  }
}

// ------------------------------------------------------------- plumbing
thread_local char g_hip_error[256] = "no HIP error recorded";

// Launch failures are read back with hipGetLastError, which also returns
// an error that an earlier, unrelated HIP call left pending in this thread.
// Such an error predates the call: it is cleared before the first launch
// so that it is not reported as this call's.
void clear_stale_hip_error() { (void)hipGetLastError(); }

int hip_fail(hipError_t e, const char* where) {
  snprintf(g_hip_error, sizeof g_hip_error, "HIP error in %s: %s", where,
           hipGetErrorString(e));
  return MMAEMU_ERR_HIP;
}

int check_model_dtype(int model, int dtype) {
  if (model != MMAEMU_MODEL_AMPERE && model != MMAEMU_MODEL_HOPPER &&
      model != MMAEMU_MODEL_LOVELACE)
    return MMAEMU_ERR_MODEL;
  if (dtype != MMAEMU_DTYPE_FP16 && dtype != MMAEMU_DTYPE_BF16 &&
      dtype != MMAEMU_DTYPE_FP8_E4M3)
    return MMAEMU_ERR_DTYPE;
  if (dtype == MMAEMU_DTYPE_FP8_E4M3 && model != MMAEMU_MODEL_HOPPER)
    return MMAEMU_ERR_UNSUPPORTED;
  return MMAEMU_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = (uintptr_t)p;
  return Range{lo, p ? lo + (uintptr_t)bytes : lo};
}

// A, B, C read-only; D and xorsum written.  D == C exactly is allowed.
int check_alias(const void* A, int64_t abytes, const void* B, int64_t bbytes,
                const void* C, const void* D, int64_t cdbytes, const void* X,
                int64_t xbytes) {
  const Range ra = range_of(A, abytes), rb = range_of(B, bbytes);
  const Range rc = range_of(C, cdbytes), rd = range_of(D, cdbytes);
  const Range rx = range_of(X, xbytes);
  if (overlap(rd, ra) || overlap(rd, rb) || overlap(rx, ra) || overlap(rx, rb) ||
      overlap(rx, rc) || overlap(rx, rd))
    return MMAEMU_ERR_ALIAS;
  if (C && C != D && overlap(rc, rd)) return MMAEMU_ERR_ALIAS;
  return MMAEMU_OK;
}

// Verify mode: A, B, C and the claimed D are read-only (they may overlap
// one another); the report and the row words are written and may overlap
// nothing.
int check_alias_verify(const void* A, int64_t abytes, const void* B, int64_t bbytes,
                       const void* C, const void* Dc, int64_t cdbytes, const void* R,
                       const void* X, int64_t xbytes) {
  const Range in[4] = {range_of(A, abytes), range_of(B, bbytes), range_of(C, cdbytes),
                       range_of(Dc, cdbytes)};
  const Range rr = range_of(R, 16), rx = range_of(X, xbytes);
  if (overlap(rr, rx)) return MMAEMU_ERR_ALIAS;
  for (const Range& r : in)
    if (overlap(rr, r) || overlap(rx, r)) return MMAEMU_ERR_ALIAS;
  return MMAEMU_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a == 0 || b == 0) {
    *out = 0;
    return true;
  }
  if (a > INT64_MAX / b) return false;
  *out = a * b;
  return true;
}

// The largest operand-image workspace one call takes: 1 GiB, or the byte
// count in MMAEMU_WORKSPACE_MAX_BYTES; 0 there, or MMAEMU_NO_WORKSPACE set,
// turns the workspace off.  Read on every call.
constexpr int64_t kDefaultWorkspaceCap = int64_t(1) << 30;

int64_t workspace_cap() {
  if (getenv("MMAEMU_NO_WORKSPACE")) return 0;
  const char* v = getenv("MMAEMU_WORKSPACE_MAX_BYTES");
  if (v && *v) {
    char* end = nullptr;
    const long long x = strtoll(v, &end, 10);
    if (end && *end == '\0' && x >= 0) return (int64_t)x;
  }
  return kDefaultWorkspaceCap;
}

// Which chain kernel is faster for an M x N output: an estimate of each
// one's time per K-step (both scale with the step count), in units of
// 10 ns, fitted on one MI355X (FP16 Ampere and E4M3 Hopper, 18 shapes from
// 1 x 4096 to 2048 x 256 and 1024 x 1024, K from 1024 to 65536):
//  * narrow kernel, one lane per output in 16 x 16 tiles:
//    max(0.74, 0.44 + 0.0013 * tiles) us, a latency floor for small shapes;
//  * tiled kernel, 4 x 4 outputs per lane in 64 x 64 blocks: 4.45 us per
//    round of 256 blocks (one per CU) up to 1024 blocks, 2.7 us per 256
//    blocks beyond (three at a time per CU).
// A few rows against a wide N (a decoding step) go to the narrow kernel
// even when M * N is large: the tiled kernel pays for whole 64-row blocks.
bool narrow_is_faster(int64_t M, int64_t N) {
  const int64_t t16 = ((M + 15) / 16) * ((N + 15) / 16);
  const int64_t b64 = ((M + 63) / 64) * ((N + 63) / 64);
  const int64_t narrow = 44 + t16 * 13 / 100 > 74 ? 44 + t16 * 13 / 100 : 74;
  const int64_t tiled = b64 <= 1024 ? 445 * ((b64 + 255) / 256) : 270 * b64 / 256;
  return narrow < tiled;
}

// MMAEMU_NARROW_BLOCKS, read on every call, replaces that estimate by a
// threshold: the narrow kernel below that many 64 x 64 blocks' worth of
// outputs (M * N / 4096), 0 never.  -1 when it is not set.
int64_t narrow_blocks() {
  const char* v = getenv("MMAEMU_NARROW_BLOCKS");
  if (v && *v) {
    char* end = nullptr;
    const long long x = strtoll(v, &end, 10);
    if (end && *end == '\0' && x >= 0) return (int64_t)x;
  }
  return -1;
}

// Stream-ordered workspace for the operand pre-pass, from one memory pool
// per device.  The pool keeps up to the default cap of freed memory cached
// (its release threshold), so repeated calls allocate no new device memory,
// and returns the rest at the next synchronisation.  A failed allocation is
// not an error: the caller falls back to the kernel that unpacks in place.
constexpr int kMaxDevices = 64;
hipMemPool_t g_pool[kMaxDevices];
std::once_flag g_pool_once[kMaxDevices];

void* workspace_alloc(int64_t bytes, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::call_once(g_pool_once[dev], [dev] {
    hipMemPoolProps props;
    memset(&props, 0, sizeof props);
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    if (hipMemPoolCreate(&g_pool[dev], &props) == hipSuccess) {
      uint64_t keep = (uint64_t)kDefaultWorkspaceCap;
      (void)hipMemPoolSetAttribute(g_pool[dev], hipMemPoolAttrReleaseThreshold, &keep);
    } else {
      g_pool[dev] = nullptr;
      (void)hipGetLastError();
    }
  });
  if (!g_pool[dev]) return nullptr;
  void* p = nullptr;
  if (hipMallocFromPoolAsync(&p, (size_t)bytes, g_pool[dev], s) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return p;
}

template <int MODEL, int DT>
hipError_t launch_gemm(const void* A, const void* B, const uint32_t* C, const Sink& out,
                       int64_t M, int64_t N, int64_t K, hipStream_t s, int64_t splits = 1) {
  // A plain chain taller than the tiled grids (65,535 blocks of 64 rows)
  // runs as row slices of that height: rows of D depend only on the same
  // rows of A and C, so a slice is the same GEMM on offset pointers.
  constexpr int64_t kSliceRows = int64_t(65535) * fastk::BM;
  if (M > kSliceRows && splits == 1 && !out.claimed && !out.accumulate &&
      gemm_fast_supported(kSliceRows, N, K)) {
    for (int64_t r0 = 0; r0 < M; r0 += kSliceRows) {
      const int64_t m = M - r0 < kSliceRows ? M - r0 : kSliceRows;
      Sink o = out;
      o.D = out.D + r0 * N;
      if (out.xorsum) o.xorsum = out.xorsum + r0;
      const hipError_t e = launch_gemm<MODEL, DT>(
          (const char*)A + r0 * K * Fmt<DT>::bytes, B, C ? C + r0 * N : nullptr, o, m, N, K,
          s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (out.xorsum && M > 0) {
    const int64_t blocks = (M + 255) / 256;
    fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(out.xorsum, M);
  }
  if (out.report) init_report_kernel<<<dim3(1), dim3(64), 0, s>>>(out.report);
  if (M == 0 || N == 0) return hipGetLastError();
  // (the narrow grid's y dimension, 16 rows a block, stays within 65,535
  // blocks, as the tiled grid's does; a taller shape runs tiled)
  const int64_t nb_env = narrow_blocks();
  if (gemm_fast_supported(M, N, K) && splits == 1 && (M + 15) / 16 <= 65535 &&
      (nb_env >= 0 ? M * N / 4096 < nb_env : narrow_is_faster(M, N))) {
    narrowk::gemm_narrow_kernel<MODEL, DT>
        <<<dim3((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16)), dim3(256), 0, s>>>(
            A, B, C, out, M, N, K, 0, K / 16);
    return hipGetLastError();
  }
  if (gemm_fast_supported(M, N, K)) {
    const int64_t nsteps = K / 16, per = nsteps / splits;
    const int64_t step_bytes = gemm_fast_workspace_bytes(M, N, 16);
    const int64_t cap = workspace_cap();
    void* ws = nullptr;
    int64_t ws_steps = 0;
    uint32_t* partials = nullptr;
    // split-K: the runs side by side when the images of all steps and one
    // M x N partial result per run fit under the cap
    const int64_t cd = M * N * 4;  // no overflow: checked with the shape
    if (splits > 1 && out.D && splits <= 65535 && cd <= cap / splits &&
        nsteps <= (cap - splits * cd) / step_bytes) {
      ws = workspace_alloc(nsteps * step_bytes + splits * cd, s);
      if (ws) {
        ws_steps = nsteps;
        partials = (uint32_t*)((char*)ws + nsteps * step_bytes);
      }
    }
    if (!ws) {
      // as many steps of operand images as the cap allows: all K/16, else
      // one split-K run's worth, else fewer (chunks)
      ws_steps = cap / step_bytes;
      if (ws_steps > nsteps) ws_steps = nsteps;
      if (ws_steps < nsteps && ws_steps > per) ws_steps = per;
      ws = ws_steps > 0 ? workspace_alloc(ws_steps * step_bytes, s) : nullptr;
    }
    gemm_fast_launch<MODEL, DT>(A, B, C, out, M, N, K, ws, ws_steps, s, splits, partials);
    if (ws) {
      // the free is ordered after the kernels; it is issued whatever the
      // launches returned, so that a failed call does not hold the memory
      const hipError_t e = hipGetLastError();
      (void)hipFreeAsync(ws, s);
      if (e != hipSuccess) return e;
    }
  } else {
    const int64_t cb = (N + 255) / 256;
    const int64_t rows = M < 32768 ? M : 32768;
    const int64_t per = K / 16 / splits;
    for (int64_t r = 0; r < splits; ++r) {
      Sink o = out;
      o.accumulate = r > 0;
      if (r + 1 < splits) o.xorsum = nullptr;
      gemm_reference_kernel<MODEL, DT><<<dim3((unsigned)cb, (unsigned)rows), dim3(256), 0, s>>>(
          A, B, r == 0 ? C : nullptr, o, M, N, K, r * per, per);
    }
  }
  return hipGetLastError();
}

template <int MODEL, int DT>
hipError_t launch_tiles(const void* A, const void* B, const uint32_t* C, uint32_t* D,
                        uint32_t* X, int64_t ntiles, hipStream_t s) {
  // one wave per four tiles, in a grid-stride loop: 7 waves per CU (the
  // LDS bound) on 256 CUs, each with several groups of tiles to overlap
  // its loads with
  const int64_t groups = (ntiles + tilek::TPW - 1) / tilek::TPW;
  const int64_t grid = groups < 1792 ? groups : 1792;
  tilek::tiles_fast_kernel<MODEL, DT>
      <<<dim3((unsigned)grid), dim3(64), 0, s>>>(A, B, C, D, X, ntiles);
  return hipGetLastError();
}

// LOVELACE runs the Ampere kernels (see the model enum in mmaemu.h).
#define MMAEMU_DISPATCH(model, dtype, FN, ...)                                  \
  ((model) == MMAEMU_MODEL_AMPERE || (model) == MMAEMU_MODEL_LOVELACE           \
       ? ((dtype) == MMAEMU_DTYPE_FP16 ? FN<kAmpere, kFP16>(__VA_ARGS__)        \
                                       : FN<kAmpere, kBF16>(__VA_ARGS__))       \
       : ((dtype) == MMAEMU_DTYPE_FP16                                          \
              ? FN<kHopper, kFP16>(__VA_ARGS__)                                 \
              : ((dtype) == MMAEMU_DTYPE_BF16 ? FN<kHopper, kBF16>(__VA_ARGS__) \
                                              : FN<kHopper, kE4M3>(__VA_ARGS__))))

// Byte sizes of a GEMM's operands; false if the shape is invalid.
struct GemmBytes {
  int64_t a, b, cd;
};

int check_gemm_shape(int dtype, int64_t M, int64_t N, int64_t K, GemmBytes* g) {
  if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return MMAEMU_ERR_SHAPE;
  const int64_t esz = dtype == MMAEMU_DTYPE_FP8_E4M3 ? 1 : 2;
  int64_t mk, kn, mn;
  if (!mul_ok(M, K, &mk) || !mul_ok(K, N, &kn) || !mul_ok(M, N, &mn) ||
      !mul_ok(mk, esz, &g->a) || !mul_ok(kn, esz, &g->b) || !mul_ok(mn, 4, &g->cd))
    return MMAEMU_ERR_SHAPE;
  if (N > (int64_t)INT32_MAX || M > (int64_t)INT32_MAX * 256) return MMAEMU_ERR_SHAPE;
  return MMAEMU_OK;
}

int gemm_impl(int model, int dtype, const void* A, const void* B, const float* C,
              float* D, int64_t M, int64_t N, int64_t K, uint32_t* xorsum,
              hipStream_t s, int64_t splits = 1) {
  int rc = check_model_dtype(model, dtype);
  if (rc) return rc;
  GemmBytes g;
  rc = check_gemm_shape(dtype, M, N, K, &g);
  if (rc) return rc;
  // split-K: a whole number of steps per run
  if (splits < 1 || (K == 0 ? splits != 1 : (K / 16) % splits != 0)) return MMAEMU_ERR_SHAPE;
  // an empty D: nothing to compute; the xorsum words of its M empty rows
  // are still written (as zeros)
  if (g.cd == 0 && !(xorsum && M > 0)) return MMAEMU_OK;
  if (g.cd > 0 && (!D || (K > 0 && (!A || !B)))) return MMAEMU_ERR_NULL;
  rc = check_alias(g.cd && K ? A : nullptr, g.a, g.cd && K ? B : nullptr, g.b,
                   g.cd ? C : nullptr, g.cd ? D : nullptr, g.cd, xorsum, xorsum ? M * 4 : 0);
  if (rc) return rc;
  const Sink out{(uint32_t*)D, xorsum, nullptr, nullptr, 0};
  clear_stale_hip_error();
  const hipError_t e = MMAEMU_DISPATCH(model, dtype, launch_gemm, A, B, (const uint32_t*)C,
                                       out, M, N, K, s, splits);
  if (e != hipSuccess) return hip_fail(e, "mma_emulate_gemm launch");
  return MMAEMU_OK;
}

int verify_impl(int model, int dtype, const void* A, const void* B, const float* C,
                const float* D_claimed, int64_t M, int64_t N, int64_t K, uint64_t* report,
                uint32_t* row_diff, hipStream_t s) {
  int rc = check_model_dtype(model, dtype);
  if (rc) return rc;
  GemmBytes g;
  rc = check_gemm_shape(dtype, M, N, K, &g);
  if (rc) return rc;
  if (!report) return MMAEMU_ERR_NULL;
  if (g.cd > 0 && (!D_claimed || (K > 0 && (!A || !B)))) return MMAEMU_ERR_NULL;
  const bool any = g.cd > 0;
  rc = check_alias_verify(any && K ? A : nullptr, g.a, any && K ? B : nullptr, g.b,
                          any ? C : nullptr, any ? D_claimed : nullptr, g.cd, report,
                          row_diff, row_diff ? M * 4 : 0);
  if (rc) return rc;
  const Sink out{nullptr, row_diff, (const uint32_t*)D_claimed, (unsigned long long*)report,
                 0};
  clear_stale_hip_error();
  const hipError_t e =
      MMAEMU_DISPATCH(model, dtype, launch_gemm, A, B, (const uint32_t*)C, out, M, N, K, s);
  if (e != hipSuccess) return hip_fail(e, "mma_verify_gemm launch");
  return MMAEMU_OK;
}

}  // namespace

extern "C" {

int mma_emulate_gemm_async(int model, int dtype, const void* A, const void* B,
                           const float* C, float* D, int64_t M, int64_t N, int64_t K,
                           uint32_t* xorsum_out, void* hip_stream) {
  return gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, (hipStream_t)hip_stream);
}

int mma_emulate_gemm(int model, int dtype, const void* A, const void* B, const float* C,
                     float* D, int64_t M, int64_t N, int64_t K, uint32_t* xorsum_out) {
  const int rc = gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, nullptr);
  if (rc) return rc;
  const hipError_t e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return hip_fail(e, "mma_emulate_gemm synchronize");
  return MMAEMU_OK;
}

int mma_emulate_gemm_splitk_async(int model, int dtype, const void* A, const void* B,
                                  const float* C, float* D, int64_t M, int64_t N, int64_t K,
                                  int64_t splits, uint32_t* xorsum_out, void* hip_stream) {
  return gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, (hipStream_t)hip_stream,
                   splits);
}

int mma_emulate_gemm_splitk(int model, int dtype, const void* A, const void* B,
                            const float* C, float* D, int64_t M, int64_t N, int64_t K,
                            int64_t splits, uint32_t* xorsum_out) {
  const int rc = gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, nullptr, splits);
  if (rc) return rc;
  const hipError_t e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return hip_fail(e, "mma_emulate_gemm_splitk synchronize");
  return MMAEMU_OK;
}

int mma_verify_gemm_async(int model, int dtype, const void* A, const void* B,
                          const float* C, const float* D_claimed, int64_t M, int64_t N,
                          int64_t K, uint64_t* report, uint32_t* row_diff_out,
                          void* hip_stream) {
  return verify_impl(model, dtype, A, B, C, D_claimed, M, N, K, report, row_diff_out,
                     (hipStream_t)hip_stream);
}

int mma_verify_gemm(int model, int dtype, const void* A, const void* B, const float* C,
                    const float* D_claimed, int64_t M, int64_t N, int64_t K, uint64_t* report,
                    uint32_t* row_diff_out) {
  const int rc =
      verify_impl(model, dtype, A, B, C, D_claimed, M, N, K, report, row_diff_out, nullptr);
  if (rc) return rc;
  const hipError_t e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return hip_fail(e, "mma_verify_gemm synchronize");
  return MMAEMU_OK;
}

int mma_emulate_tiles(int model, int dtype, const void* A, const void* B, const float* C,
                      float* D, int64_t ntiles, uint32_t* xorsum_out, void* hip_stream) {
  int rc = check_model_dtype(model, dtype);
  if (rc) return rc;
  if (ntiles < 0 || ntiles > (int64_t)INT32_MAX) return MMAEMU_ERR_SHAPE;
  if (ntiles == 0) return MMAEMU_OK;
  if (!A || !B || !D) return MMAEMU_ERR_NULL;
  const int64_t esz = dtype == MMAEMU_DTYPE_FP8_E4M3 ? 1 : 2;
  rc = check_alias(A, ntiles * 256 * esz, B, ntiles * 256 * esz, C, D, ntiles * 1024,
                   xorsum_out, xorsum_out ? ntiles * 4 : 0);
  if (rc) return rc;
  clear_stale_hip_error();
  const hipError_t e =
      MMAEMU_DISPATCH(model, dtype, launch_tiles, A, B, (const uint32_t*)C, (uint32_t*)D,
                      xorsum_out, ntiles, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "mma_emulate_tiles launch");
  return MMAEMU_OK;
}

const char* mma_emulate_strerror(int code) {
  switch (code) {
    case MMAEMU_OK: return "ok";
    case MMAEMU_ERR_MODEL: return "unknown model";
    case MMAEMU_ERR_DTYPE: return "unknown dtype";
    case MMAEMU_ERR_UNSUPPORTED: return "FP8 E4M3 exists only with the Hopper model";
    case MMAEMU_ERR_SHAPE: return "bad shape (negative, K not a multiple of 16, or too large)";
    case MMAEMU_ERR_NULL: return "a required pointer is NULL";
    case MMAEMU_ERR_ALIAS: return "buffers overlap (only D == C is allowed)";
    case MMAEMU_ERR_HIP: return g_hip_error;
    default: return "unknown error code";
  }
}

int mma_emulate_spec_version(void) { return kSpecVersion; }

}  // extern "C"
