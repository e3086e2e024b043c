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
#include "gemm_spread.h"
#include "tiles_fast.h"

using namespace mmaemu;

namespace {

constexpr int kSpecVersion = 1;

// --------------------------------------------------- reference GEMM path
// One lane per output, the chained steps read straight from global memory.
// Kept as the simple, fully general path (any shape, any input bits).  It
// chains the ns chain positions that start at s0; position p applies K-step
// step_at(order, p).
template <int MODEL, int DT>
__global__ __launch_bounds__(256) void gemm_reference_kernel(
    const void* __restrict__ A, const void* __restrict__ B, const uint32_t* C, Sink out,
    int64_t M, int64_t N, int64_t K, int64_t s0, int64_t ns,
    const int32_t* __restrict__ order) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = col < N;
  uint32_t nbad = 0;
  unsigned long long first = ~0ull;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    uint32_t c = 0, x = 0;
    if (live) {
      c = C ? C[row * N + col] : 0u;
      for (int64_t p = s0; p < s0 + ns; ++p) {
        const int64_t t = step_at(order, p, K / 16);
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

// A, B, C and the step order O read-only; D and xorsum written.  D == C
// exactly is allowed.
int check_alias(const void* A, int64_t abytes, const void* B, int64_t bbytes,
                const void* C, const void* D, int64_t cdbytes, const void* X,
                int64_t xbytes, const void* O = nullptr, int64_t obytes = 0) {
  const Range ra = range_of(A, abytes), rb = range_of(B, bbytes);
  const Range rc = range_of(C, cdbytes), rd = range_of(D, cdbytes);
  const Range rx = range_of(X, xbytes), ro = range_of(O, obytes);
  if (overlap(rd, ra) || overlap(rd, rb) || overlap(rx, ra) || overlap(rx, rb) ||
      overlap(rx, rc) || overlap(rx, rd) || overlap(rd, ro) || overlap(rx, ro))
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

// Every pointer at the alignment of its elements: the kernels read and
// write whole elements, and update the xorsum words (32-bit) and the
// report (64-bit) with atomics, which need natural alignment.  NULL passes.
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_align(int dtype, const void* A, const void* B, const void* C, const void* D,
                const void* X, const void* O = nullptr, const void* R = nullptr) {
  const uintptr_t esz = dtype == MMAEMU_DTYPE_FP8_E4M3 ? 1 : 2;
  if (!aligned(A, esz) || !aligned(B, esz) || !aligned(C, 4) || !aligned(D, 4) ||
      !aligned(X, 4) || !aligned(O, 4) || !aligned(R, 8))
    return MMAEMU_ERR_ALIGN;
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
// per device, created on first use.  Its release threshold is 0: memory that
// a call frees (in stream order, after its kernels) goes back to the device
// at the next synchronisation of the stream, an event or the device, and
// the blocking entry points trim the pool after their own synchronisation,
// so no workspace memory stays held between synchronised calls.  Freed
// blocks are still reused by later calls enqueued before that
// synchronisation.  A failed allocation is not an error: the caller falls
// back to the kernel that builds its images in LDS.
constexpr int kMaxDevices = 64;
hipMemPool_t g_pool[kMaxDevices];
std::once_flag g_pool_once[kMaxDevices];

hipMemPool_t pool_of(int dev) {
  std::call_once(g_pool_once[dev], [dev] {
    hipMemPoolProps props;
    memset(&props, 0, sizeof props);
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    if (hipMemPoolCreate(&g_pool[dev], &props) == hipSuccess) {
      uint64_t keep = 0;
      (void)hipMemPoolSetAttribute(g_pool[dev], hipMemPoolAttrReleaseThreshold, &keep);
    } else {
      g_pool[dev] = nullptr;
      (void)hipGetLastError();
    }
  });
  return g_pool[dev];
}

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return -1;
  }
  return dev;
}

void* workspace_alloc(int64_t bytes, hipStream_t s) {
  const int dev = current_device();
  if (dev < 0) return nullptr;
  hipMemPool_t pool = pool_of(dev);
  if (!pool) return nullptr;
  void* p = nullptr;
  if (hipMallocFromPoolAsync(&p, (size_t)bytes, pool, s) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return p;
}

// After a blocking call's synchronisation: return what the pool of the
// current device still holds (nothing of it is in use any more).
void trim_workspace_pool() {
  const int dev = current_device();
  if (dev < 0) return;
  hipMemPool_t pool = pool_of(dev);
  if (pool && hipMemPoolTrimTo(pool, 0) != hipSuccess) (void)hipGetLastError();
}

// The workspace of mma_emulate_gemm_noalloc_async: a fixed array of device
// memory, one copy per GPU the library runs on, held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress (while
// that device is current) and only that address is ever handed to a kernel.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The device address of the current device's scratch array (NULL and the
// HIP error if it cannot be taken).
void* scratch_of(int dev, hipError_t* err) {
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    g_scratch[dev] = p;
    g_scratch_err[dev] = e;
  });
  *err = g_scratch_err[dev];
  return g_scratch[dev];
}

// Where a GEMM's workspace comes from: the pool (fixed == NULL), or a buffer
// of fixed_bytes that the caller of launch_gemm provides.
struct WorkspaceSource {
  void* fixed;
  int64_t fixed_bytes;
};

// Everything launch_gemm needs besides the operands: the split-K run count,
// the step order (NULL: forward) and the workspace source.
struct Schedule {
  int64_t splits;
  const int32_t* order;
  WorkspaceSource ws;
};

// A plain chain taller than the tiled grids (65,535 blocks of 64 rows)
// runs as row slices of that height: rows of D depend only on the same
// rows of A and C, so a slice is the same GEMM on offset pointers.
constexpr int64_t kSliceRows = int64_t(65535) * fastk::BM;

bool row_slices(int64_t M, int64_t N, int64_t K, int64_t splits, const Sink& out) {
  return M > kSliceRows && splits == 1 && !out.claimed && !out.accumulate &&
         gemm_fast_supported(kSliceRows, N, K);
}

// The narrow kernel takes a plain chain that it is estimated to run faster
// (or that MMAEMU_NARROW_BLOCKS sends to it); its grid's y dimension, 16
// rows a block, stays within 65,535 blocks, as the tiled grid's does.
bool takes_narrow(int64_t M, int64_t N, int64_t K, int64_t splits) {
  if (!gemm_fast_supported(M, N, K) || splits != 1 || (M + 15) / 16 > 65535) return false;
  const int64_t nb_env = narrow_blocks();
  return nb_env >= 0 ? M * N / 4096 < nb_env : narrow_is_faster(M, N);
}

// MMAEMU_SPREAD_LANES, read on every call: 0 never runs the spread kernel,
// 2 or 4 runs it with that many lanes per output wherever the narrow kernel
// would run; -1 when it is not set (or set to anything else).
int spread_env() {
  const char* v = getenv("MMAEMU_SPREAD_LANES");
  if (v && (!strcmp(v, "0") || !strcmp(v, "2") || !strcmp(v, "4"))) return atoi(v);
  return -1;
}

// Lanes per output of the spread kernel for a chain that the narrow kernel
// would take (0: the narrow kernel itself).  The narrow kernel runs four
// waves per 16 x 16 tile; at two waves per SIMD or fewer (2048 waves on the
// 256 CUs) its SIMDs mostly wait on the dependent instructions of one
// wave's step, and two lanes per output (twice the waves, half the products
// per lane) win: measured on MI355X, 256 x 256 x 65536 FP16 Ampere 3.33 ->
// 2.15 ms, 48 x 48 x 65536 3.23 -> 1.40 ms, 128 x 1024 x 16384 1.12 ->
// 1.00 ms (E4M3 Hopper 3.17 -> 1.94, 3.15 -> 1.09 and 1.07 -> 0.86 ms);
// at 4096 waves (512 x 512) the two are even, beyond it the narrow kernel
// wins.  Four lanes (4-row tiles) while that still makes at most one wave
// per SIMD: a lone wave's step is shorter with four products per lane than
// with eight (48 x 48 x 65536 E4M3 Hopper 1.40 -> 1.09 ms).
int spread_lanes(int64_t M, int64_t N) {
  const int e = spread_env();
  if (e >= 0) return e;
  const int64_t waves = 4 * ((M + 15) / 16) * ((N + 15) / 16);
  if (waves > 2048) return 0;
  return 4 * ((M + 3) / 4) * ((N + 15) / 16) <= 1024 ? 4 : 2;
}

// The spread kernel's grids: (N / 16, rows / (16 / L)) and the pre-pass's
// (positions, images / 64).
bool spread_supported(int64_t M, int64_t N, int L) {
  return (M + 3) / 4 <= 65535 && (M + 63) / 64 <= 65535 && (N + 63) / 64 <= 65535 &&
         (L == 2 || L == 4);
}

template <int MODEL, int DT, int L>
void spread_launch(const void* A, const void* B, const uint32_t* C, const Sink& out,
                   int64_t M, int64_t N, int64_t K, void* ws, int64_t ws_steps, hipStream_t s,
                   const int32_t* order) {
  spreadk::gemm_spread_launch<MODEL, DT, L>(A, B, C, out, M, N, K, ws, ws_steps, s, order);
}

// The workspace one K-step of a plain chain needs on the kernel the
// library picks for it: the operand images of the tiled kernel, else 0 (the
// narrow kernel needs none, and the spread kernel falls back to it).
int64_t chain_step_bytes(int64_t M, int64_t N, int64_t K, const Sink& out) {
  if (M == 0 || N == 0) return 0;
  if (row_slices(M, N, K, 1, out)) return gemm_fast_workspace_bytes(kSliceRows, N, 16);
  if (takes_narrow(M, N, K, 1) || !gemm_fast_supported(M, N, K)) return 0;
  return gemm_fast_workspace_bytes(M, N, 16);
}

template <int MODEL, int DT>
hipError_t launch_gemm(const void* A, const void* B, const uint32_t* C, const Sink& out,
                       int64_t M, int64_t N, int64_t K, hipStream_t s, const Schedule& sch) {
  const int64_t splits = sch.splits;
  const int32_t* const order = sch.order;
  if (row_slices(M, N, K, splits, out)) {
    for (int64_t r0 = 0; r0 < M; r0 += kSliceRows) {
      const int64_t m = M - r0 < kSliceRows ? M - r0 : kSliceRows;
      Sink o = out;
      o.D = out.D + r0 * N;
      if (out.xorsum) o.xorsum = out.xorsum + r0;
      const hipError_t e = launch_gemm<MODEL, DT>(
          (const char*)A + r0 * K * Fmt<DT>::bytes, B, C ? C + r0 * N : nullptr, o, m, N, K,
          s, sch);
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
  if (takes_narrow(M, N, K, splits)) {
    // the spread kernel when the workspace holds its images (all K-steps'
    // for the audit compare, which cannot restart from D), else the narrow one
    const int L = spread_lanes(M, N);
    if (L && spread_supported(M, N, L)) {
      const int64_t T = K / 16;
      const int64_t step_bytes = L == 2 ? spreadk::spread_step_bytes<2>(M, N)
                                        : spreadk::spread_step_bytes<4>(M, N);
      const bool fixed = sch.ws.fixed != nullptr;
      const int64_t cap = fixed ? sch.ws.fixed_bytes : workspace_cap();
      int64_t ws_steps = cap / step_bytes < T ? cap / step_bytes : T;
      if (ws_steps < T && (out.claimed || out.accumulate || !out.D)) ws_steps = 0;
      void* ws = nullptr;
      if (ws_steps > 0) ws = fixed ? sch.ws.fixed : workspace_alloc(ws_steps * step_bytes, s);
      if (ws) {
        if (L == 2) {
          spread_launch<MODEL, DT, 2>(A, B, C, out, M, N, K, ws, ws_steps, s, order);
        } else {
          spread_launch<MODEL, DT, 4>(A, B, C, out, M, N, K, ws, ws_steps, s, order);
        }
        const hipError_t e = hipGetLastError();
        if (!fixed) (void)hipFreeAsync(ws, s);
        return e;
      }
    }
    const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16));
    {
      // the narrow kernel with A from row images (the spread kernel's
      // pre-pass, rows padded to 16) when the workspace holds all K-steps'
      const int64_t T = K / 16, ma = (M + 15) / 16 * 16;
      const int64_t bytes = ma * spreadk::IW * 4 * T;
      const bool fixed = sch.ws.fixed != nullptr;
      const int64_t cap = fixed ? sch.ws.fixed_bytes : workspace_cap();
      void* ws = nullptr;
      if (bytes <= cap && (ma + 63) / 64 <= 65535)
        ws = fixed ? sch.ws.fixed : workspace_alloc(bytes, s);
      if (ws) {
        spreadk::spread_unpack_kernel<MODEL, DT, false>
            <<<dim3((unsigned)T, (unsigned)((ma + 63) / 64)), dim3(64), 0, s>>>(
                A, M, K, N, 0, order, (uint32_t*)ws, ma);
        narrowk::gemm_narrow_kernel<MODEL, DT, true><<<grid, dim3(256), 0, s>>>(
            A, B, C, out, M, N, K, 0, T, order, (const uint32_t*)ws, ma, 0);
        const hipError_t e = hipGetLastError();
        if (!fixed) (void)hipFreeAsync(ws, s);
        return e;
      }
    }
    narrowk::gemm_narrow_kernel<MODEL, DT><<<grid, dim3(256), 0, s>>>(A, B, C, out, M, N, K, 0,
                                                                     K / 16, order);
    return hipGetLastError();
  }
  if (gemm_fast_supported(M, N, K)) {
    const int64_t nsteps = K / 16, per = nsteps / splits;
    const int64_t step_bytes = gemm_fast_workspace_bytes(M, N, 16);
    const bool fixed = sch.ws.fixed != nullptr;
    const int64_t cap = fixed ? sch.ws.fixed_bytes : workspace_cap();
    auto take = [&](int64_t bytes) -> void* {
      if (fixed) return bytes <= sch.ws.fixed_bytes ? sch.ws.fixed : nullptr;
      return workspace_alloc(bytes, s);
    };
    void* ws = nullptr;
    int64_t ws_steps = 0;
    uint32_t* partials = nullptr;
    // split-K: the runs side by side when the images of all steps and one
    // M x N partial result per run fit under the cap
    const int64_t cd = M * N * 4;  // no overflow: checked with the shape
    if (splits > 1 && out.D && splits <= 65535 && cd <= cap / splits &&
        nsteps <= (cap - splits * cd) / step_bytes) {
      ws = take(nsteps * step_bytes + splits * cd);
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
      ws = ws_steps > 0 ? take(ws_steps * step_bytes) : nullptr;
    }
    gemm_fast_launch<MODEL, DT>(A, B, C, out, M, N, K, ws, ws_steps, s, splits, partials,
                                order);
    if (ws && !fixed) {
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
          A, B, r == 0 ? C : nullptr, o, M, N, K, r * per, per, order);
    }
  }
  return hipGetLastError();
}

template <int MODEL, int DT>
hipError_t launch_tiles(const void* A, const void* B, const uint32_t* C, uint32_t* D,
                        uint32_t* X, int64_t ntiles, hipStream_t s) {
  // one wave per two tiles: one workgroup per CU (256 of them), of as
  // many waves as a CU holds at once, each workgroup sharing out an equal
  // part of the groups of tiles among its waves.  The kernel counts tiles
  // in 32 bits: a larger batch runs as launches of 2^30 tiles each, every
  // tile being independent.
  const int64_t esz = DT == kE4M3 ? 1 : 2;
  constexpr int64_t kChunk = int64_t(1) << 30;
  for (int64_t t = 0; t < ntiles; t += kChunk) {
    const int64_t n = ntiles - t < kChunk ? ntiles - t : kChunk;
    const int64_t groups = (n + tilek::TPW - 1) / tilek::TPW;
    const int64_t grid = groups < 256 ? groups : 256;
    tilek::tiles_fast_kernel<MODEL, DT>
        <<<dim3((unsigned)grid), dim3(64 * tilek::kWavesPerCU<MODEL>), 0, s>>>(
        (const char*)A + t * 256 * esz, (const char*)B + t * 256 * esz, C ? C + t * 256 : nullptr,
        D + t * 256, X ? X + t : nullptr, (uint32_t)n);
  }
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

// Every argument check of a GEMM call, before anything touches the device.
// Sets *nothing when the call has nothing to do.
int gemm_check(int model, int dtype, const void* A, const void* B, const float* C, float* D,
               int64_t M, int64_t N, int64_t K, uint32_t* xorsum, const Schedule& sch,
               bool* nothing) {
  *nothing = false;
  int rc = check_model_dtype(model, dtype);
  if (rc) return rc;
  GemmBytes g;
  rc = check_gemm_shape(dtype, M, N, K, &g);
  if (rc) return rc;
  const int64_t splits = sch.splits;
  // split-K: a whole number of steps per run
  if (splits < 1 || (K == 0 ? splits != 1 : (K / 16) % splits != 0)) return MMAEMU_ERR_SHAPE;
  // an empty D: nothing to compute; the xorsum words of its M empty rows
  // are still written (as zeros)
  if (g.cd == 0 && !(xorsum && M > 0)) {
    *nothing = true;
    return MMAEMU_OK;
  }
  if (g.cd > 0 && (!D || (K > 0 && (!A || !B)))) return MMAEMU_ERR_NULL;
  // the step order is read only when there are steps and outputs
  const int32_t* order = g.cd > 0 && K > 0 ? sch.order : nullptr;
  rc = check_align(dtype, A, B, C, D, xorsum, order);
  if (rc) return rc;
  return check_alias(g.cd && K ? A : nullptr, g.a, g.cd && K ? B : nullptr, g.b,
                     g.cd ? C : nullptr, g.cd ? D : nullptr, g.cd, xorsum, xorsum ? M * 4 : 0,
                     order, order ? K / 16 * 4 : 0);
}

int gemm_impl(int model, int dtype, const void* A, const void* B, const float* C,
              float* D, int64_t M, int64_t N, int64_t K, uint32_t* xorsum,
              hipStream_t s, const Schedule& sch, const char* where) {
  bool nothing = false;
  const int rc = gemm_check(model, dtype, A, B, C, D, M, N, K, xorsum, sch, &nothing);
  if (rc || nothing) return rc;
  const Sink out{(uint32_t*)D, xorsum, nullptr, nullptr, 0};
  Schedule run = sch;
  if (M * N == 0 || K == 0) run.order = nullptr;
  clear_stale_hip_error();
  const hipError_t e = MMAEMU_DISPATCH(model, dtype, launch_gemm, A, B, (const uint32_t*)C,
                                       out, M, N, K, s, run);
  if (e != hipSuccess) return hip_fail(e, where);
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
  rc = check_align(dtype, A, B, C, D_claimed, row_diff, nullptr, report);
  if (rc) return rc;
  const bool any = g.cd > 0;
  rc = check_alias_verify(any && K ? A : nullptr, g.a, any && K ? B : nullptr, g.b,
                          any ? C : nullptr, any ? D_claimed : nullptr, g.cd, report,
                          row_diff, row_diff ? M * 4 : 0);
  if (rc) return rc;
  const Sink out{nullptr, row_diff, (const uint32_t*)D_claimed, (unsigned long long*)report,
                 0};
  const Schedule sch{1, nullptr, {nullptr, 0}};
  clear_stale_hip_error();
  const hipError_t e =
      MMAEMU_DISPATCH(model, dtype, launch_gemm, A, B, (const uint32_t*)C, out, M, N, K, s, sch);
  if (e != hipSuccess) return hip_fail(e, "mma_verify_gemm launch");
  return MMAEMU_OK;
}

// The end of a blocking call: synchronise the null stream, then hand the
// workspace pool's memory back.
int finish_blocking(const char* where) {
  const hipError_t e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return hip_fail(e, where);
  trim_workspace_pool();
  return MMAEMU_OK;
}

const Schedule kPlain{1, nullptr, {nullptr, 0}};

// mma_emulate_gemm_async on the static scratch array instead of the pool.
int gemm_noalloc(int model, int dtype, const void* A, const void* B, const float* C, float* D,
                 int64_t M, int64_t N, int64_t K, uint32_t* xorsum, hipStream_t s) {
  bool nothing = false;
  const int rc = gemm_check(model, dtype, A, B, C, D, M, N, K, xorsum, kPlain, &nothing);
  if (rc || nothing) return rc;
  // the same decision the launch makes: reject a shape whose chain needs
  // more than the scratch for even one K-step of operand images
  const Sink probe{(uint32_t*)D, xorsum, nullptr, nullptr, 0};
  if (K > 0 && chain_step_bytes(M, N, K, probe) > kScratchBytes) return MMAEMU_ERR_SCRATCH;
  const int dev = current_device();
  if (dev < 0) return hip_fail(hipErrorNoDevice, "mma_emulate_gemm_noalloc_async");
  hipError_t e = hipSuccess;
  void* ws = scratch_of(dev, &e);
  if (!ws) return hip_fail(e, "mma_emulate_gemm_noalloc_async: scratch address");
  const Schedule sch{1, nullptr, {ws, kScratchBytes}};
  return gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum, s, sch,
                   "mma_emulate_gemm_noalloc_async launch");
}

}  // namespace

extern "C" {

int mma_emulate_gemm_async(int model, int dtype, const void* A, const void* B,
                           const float* C, float* D, int64_t M, int64_t N, int64_t K,
                           uint32_t* xorsum_out, void* hip_stream) {
  return gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, (hipStream_t)hip_stream,
                   kPlain, "mma_emulate_gemm launch");
}

int mma_emulate_gemm(int model, int dtype, const void* A, const void* B, const float* C,
                     float* D, int64_t M, int64_t N, int64_t K, uint32_t* xorsum_out) {
  const int rc = gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, nullptr, kPlain,
                           "mma_emulate_gemm launch");
  if (rc) return rc;
  return finish_blocking("mma_emulate_gemm synchronize");
}

int mma_emulate_gemm_noalloc_async(int model, int dtype, const void* A, const void* B,
                                   const float* C, float* D, int64_t M, int64_t N, int64_t K,
                                   uint32_t* xorsum_out, void* hip_stream) {
  return gemm_noalloc(model, dtype, A, B, C, D, M, N, K, xorsum_out, (hipStream_t)hip_stream);
}

int mma_emulate_gemm_splitk_async(int model, int dtype, const void* A, const void* B,
                                  const float* C, float* D, int64_t M, int64_t N, int64_t K,
                                  int64_t splits, uint32_t* xorsum_out, void* hip_stream) {
  const Schedule sch{splits, nullptr, {nullptr, 0}};
  return gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, (hipStream_t)hip_stream,
                   sch, "mma_emulate_gemm_splitk launch");
}

int mma_emulate_gemm_splitk(int model, int dtype, const void* A, const void* B,
                            const float* C, float* D, int64_t M, int64_t N, int64_t K,
                            int64_t splits, uint32_t* xorsum_out) {
  const Schedule sch{splits, nullptr, {nullptr, 0}};
  const int rc = gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, nullptr, sch,
                           "mma_emulate_gemm_splitk launch");
  if (rc) return rc;
  return finish_blocking("mma_emulate_gemm_splitk synchronize");
}

int mma_emulate_gemm_ordered_async(int model, int dtype, const void* A, const void* B,
                                   const float* C, float* D, int64_t M, int64_t N, int64_t K,
                                   const int32_t* order, uint32_t* xorsum_out,
                                   void* hip_stream) {
  const Schedule sch{1, order, {nullptr, 0}};
  return gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, (hipStream_t)hip_stream,
                   sch, "mma_emulate_gemm_ordered launch");
}

int mma_emulate_gemm_ordered(int model, int dtype, const void* A, const void* B,
                             const float* C, float* D, int64_t M, int64_t N, int64_t K,
                             const int32_t* order, uint32_t* xorsum_out) {
  const Schedule sch{1, order, {nullptr, 0}};
  const int rc = gemm_impl(model, dtype, A, B, C, D, M, N, K, xorsum_out, nullptr, sch,
                           "mma_emulate_gemm_ordered launch");
  if (rc) return rc;
  return finish_blocking("mma_emulate_gemm_ordered synchronize");
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
  return finish_blocking("mma_verify_gemm synchronize");
}

int mma_emulate_tiles(int model, int dtype, const void* A, const void* B, const float* C,
                      float* D, int64_t ntiles, uint32_t* xorsum_out, void* hip_stream) {
  int rc = check_model_dtype(model, dtype);
  if (rc) return rc;
  if (ntiles < 0 || ntiles > (int64_t)INT32_MAX) return MMAEMU_ERR_SHAPE;
  if (ntiles == 0) return MMAEMU_OK;
  if (!A || !B || !D) return MMAEMU_ERR_NULL;
  rc = check_align(dtype, A, B, C, D, xorsum_out);
  if (rc) return rc;
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

int mma_emulate_workspace_held(int device, uint64_t* bytes_out) {
  if (!bytes_out) return MMAEMU_ERR_NULL;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    return hip_fail(e == hipSuccess ? hipErrorNoDevice : e, "mma_emulate_workspace_held");
  }
  if (device < 0 || device >= count || device >= kMaxDevices)
    return hip_fail(hipErrorInvalidDevice, "mma_emulate_workspace_held");
  *bytes_out = 0;
  hipMemPool_t pool = pool_of(device);
  if (!pool) return MMAEMU_OK;
  uint64_t v = 0;
  const hipError_t e = hipMemPoolGetAttribute(pool, hipMemPoolAttrReservedMemCurrent, &v);
  if (e != hipSuccess) return hip_fail(e, "mma_emulate_workspace_held");
  *bytes_out = v;
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
    case MMAEMU_ERR_SCRATCH:
      return "the chain needs more than the 64 MiB static scratch for one K-step of "
             "operand images (ceil(M/64) + ceil(N/64) > 5461)";
    case MMAEMU_ERR_ALIGN:
      return "a pointer is not aligned to its elements (codes 2 bytes for FP16/BF16; "
             "C, D, xorsum and row words, step order 4 bytes; report 8 bytes)";
    default: return "unknown error code";
  }
}

int mma_emulate_spec_version(void) { return kSpecVersion; }

}  // extern "C"
