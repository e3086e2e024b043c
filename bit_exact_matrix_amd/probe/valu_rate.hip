// valu_rate.hip -- libvalurate.so: an issue-rate probe of the 32-bit VALU
// instructions the emulation's hot loop is built from, to check the VALU
// roofline peak (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3e12 lane
// operations per second) against measurement.  Measurement only: the
// emulation does not use this library.
//
// Each lane runs eight independent dependency chains of one instruction,
// 32 instructions per loop iteration; a grid of many waves per SIMD hides
// the chains' latency, so the loop runs at the instruction's issue rate.
// One more probe runs the hot loop's own pass-2 mix instead (per two
// products: two exact products, two alignment shifts, one of them reading
// its distance from a high word, two sign-and-accumulates and the
// saturating packed add of both distances): 7 instructions per chain step,
// 224 per loop iteration.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

enum {
  OP_ADD = 0,    // v_add_u32
  OP_MAD24,      // v_mad_i32_i24
  OP_XAD,        // v_xad_u32
  OP_ASHR,       // v_ashrrev_i32
  OP_PK_ADD,     // v_pk_add_u16 (two 16-bit lanes per slot)
  OP_PK_MIN3,    // v_pk_minimum3_f16
  OP_BCNT,       // v_bcnt_u32_b32
  OP_FFBH,       // v_ffbh_u32
  OP_ADD_E64,    // v_add_u32 in its 64-bit (VOP3) encoding
  OP_ASHR_SDWA,  // v_ashrrev_i32 with the shift read from a register's high word
  OP_XOR,        // v_xor_b32
  OP_MUL24,      // v_mul_i32_i24
  OP_LSHL,       // v_lshlrev_b32
  OP_MAX,        // v_max_i32
  OP_AND_OR,     // v_and_or_b32
  OP_PERM,       // v_perm_b32
  OP_PASS2_MIX,  // the hot loop's pass-2 sequence (7 instructions)
  NOPS
};
const char* const kNames[NOPS] = {
    "v_add_u32",      "v_mad_i32_i24",      "v_xad_u32",       "v_ashrrev_i32",
    "v_pk_add_u16",   "v_pk_minimum3_f16",  "v_bcnt_u32_b32",  "v_ffbh_u32",
    "v_add_u32_e64",  "v_ashrrev_i32_sdwa", "v_xor_b32",       "v_mul_i32_i24",
    "v_lshlrev_b32",  "v_max_i32",          "v_and_or_b32",    "v_perm_b32",
    "pass2_mix"};
// instructions per chain step
constexpr int kInsts[NOPS] = {1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 7};

template <int OP>
__device__ __forceinline__ void step(uint32_t& a, uint32_t b, uint32_t c) {
  if constexpr (OP == OP_ADD) {
    asm volatile("v_add_u32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_MAD24) {
    asm volatile("v_mad_i32_i24 %0, %0, %1, %2" : "+v"(a) : "v"(b), "v"(c));
  } else if constexpr (OP == OP_XAD) {
    asm volatile("v_xad_u32 %0, %0, %1, %2" : "+v"(a) : "v"(b), "v"(c));
  } else if constexpr (OP == OP_ASHR) {
    asm volatile("v_ashrrev_i32 %0, %1, %0" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_PK_ADD) {
    asm volatile("v_pk_add_u16 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_PK_MIN3) {
    asm volatile("v_pk_minimum3_f16 %0, %0, %1, %2" : "+v"(a) : "v"(b), "v"(c));
  } else if constexpr (OP == OP_BCNT) {
    asm volatile("v_bcnt_u32_b32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_FFBH) {
    asm volatile("v_ffbh_u32 %0, %0" : "+v"(a));
  } else if constexpr (OP == OP_ADD_E64) {
    asm volatile("v_add_u32_e64 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_ASHR_SDWA) {
    asm volatile(
        "v_ashrrev_i32_sdwa %0, %1, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 "
        "src1_sel:DWORD"
        : "+v"(a)
        : "v"(b));
  } else if constexpr (OP == OP_XOR) {
    asm volatile("v_xor_b32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_MUL24) {
    asm volatile("v_mul_i32_i24 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_LSHL) {
    asm volatile("v_lshlrev_b32 %0, %1, %0" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_MAX) {
    asm volatile("v_max_i32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == OP_AND_OR) {
    asm volatile("v_and_or_b32 %0, %0, %1, %2" : "+v"(a) : "v"(b), "v"(c));
  } else if constexpr (OP == OP_PASS2_MIX) {
    asm volatile(
        "v_mad_i32_i24 %0, %0, %1, %2\n"
        "v_ashrrev_i32 %0, %1, %0\n"
        "v_xad_u32 %0, %0, %1, %2\n"
        "v_mad_i32_i24 %0, %0, %1, %2\n"
        "v_ashrrev_i32_sdwa %0, %1, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 "
        "src1_sel:DWORD\n"
        "v_xad_u32 %0, %0, %1, %2\n"
        "v_pk_add_u16 %0, %0, %1 clamp"
        : "+v"(a)
        : "v"(b), "v"(c));
  } else {
    asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(a) : "v"(b), "v"(c));
  }
}

template <int OP>
__global__ __launch_bounds__(256) void rate_kernel(uint32_t* out, int64_t iters) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  uint32_t a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = t * 2654435761u + (uint32_t)i;
  const uint32_t b = t | 1u, c = 0x3C003C00u ^ t;
  for (int64_t n = 0; n < iters; ++n) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) step<OP>(a[i], b, c);
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) x ^= a[i];
  out[t] = x;
}

template <int OP>
hipError_t launch(uint32_t* out, int64_t iters, int64_t blocks, hipStream_t s) {
  rate_kernel<OP><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(out, iters);
  return hipGetLastError();
}

hipError_t launch_op(int op, uint32_t* out, int64_t iters, int64_t blocks, hipStream_t s) {
  switch (op) {
    case OP_ADD: return launch<OP_ADD>(out, iters, blocks, s);
    case OP_MAD24: return launch<OP_MAD24>(out, iters, blocks, s);
    case OP_XAD: return launch<OP_XAD>(out, iters, blocks, s);
    case OP_ASHR: return launch<OP_ASHR>(out, iters, blocks, s);
    case OP_PK_ADD: return launch<OP_PK_ADD>(out, iters, blocks, s);
    case OP_PK_MIN3: return launch<OP_PK_MIN3>(out, iters, blocks, s);
    case OP_BCNT: return launch<OP_BCNT>(out, iters, blocks, s);
    case OP_FFBH: return launch<OP_FFBH>(out, iters, blocks, s);
    case OP_ADD_E64: return launch<OP_ADD_E64>(out, iters, blocks, s);
    case OP_ASHR_SDWA: return launch<OP_ASHR_SDWA>(out, iters, blocks, s);
    case OP_XOR: return launch<OP_XOR>(out, iters, blocks, s);
    case OP_MUL24: return launch<OP_MUL24>(out, iters, blocks, s);
    case OP_LSHL: return launch<OP_LSHL>(out, iters, blocks, s);
    case OP_MAX: return launch<OP_MAX>(out, iters, blocks, s);
    case OP_AND_OR: return launch<OP_AND_OR>(out, iters, blocks, s);
    case OP_PASS2_MIX: return launch<OP_PASS2_MIX>(out, iters, blocks, s);
    default: return launch<OP_PERM>(out, iters, blocks, s);
  }
}

}  // namespace

extern "C" {

int valu_rate_nops(void) { return NOPS; }

const char* valu_rate_name(int op) { return op >= 0 && op < NOPS ? kNames[op] : "?"; }

// Instructions per chain step of probe `op` (each lane runs 32 * iters
// steps): 1 for a single instruction, 7 for the pass-2 mix, 0 if unknown.
int valu_rate_insts(int op) { return op >= 0 && op < NOPS ? kInsts[op] : 0; }

// Times `reps` launches of the probe for instruction `op` (blocks x 256
// lanes, each lane 32 * iters chain steps) after one warm-up launch, on
// the current device's null stream.  *best_ms receives the fastest launch.
// Returns 0, -1 for bad arguments, -2 for a HIP error.
int valu_rate_run(int op, int64_t iters, int64_t blocks, int reps, double* best_ms) {
  if (op < 0 || op >= NOPS || iters < 1 || blocks < 1 || blocks > (1 << 30) || reps < 1 ||
      !best_ms)
    return -1;
  uint32_t* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  float best = -1.0f;
  if (hipMalloc((void**)&out, (size_t)blocks * 256 * sizeof(uint32_t)) != hipSuccess ||
      hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    rc = -2;
  } else if (launch_op(op, out, iters, blocks, nullptr) != hipSuccess) {
    rc = -2;
  } else {
    for (int r = 0; r < reps && rc == 0; ++r) {
      float ms = 0.0f;
      if (hipEventRecord(e0, nullptr) != hipSuccess ||
          launch_op(op, out, iters, blocks, nullptr) != hipSuccess ||
          hipEventRecord(e1, nullptr) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
          hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
        rc = -2;
      } else if (best < 0.0f || ms < best) {
        best = ms;
      }
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (rc == 0) *best_ms = best;
  return rc;
}

}  // extern "C"
