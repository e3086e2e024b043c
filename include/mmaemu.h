/*
 * mmaemu.h -- C ABI of the MI355X bit-exact tile-MMA emulator (libmmaemu.so).
 *
 * WHAT IT COMPUTES
 *   D = C + A*B, built from chained 16x16x16 matrix-multiply-accumulate
 *   steps, each rounded the way the Hawkeye study recovered for NVIDIA
 *   tensor cores ("Hawkeye: Reproducing GPU-Level Non-Determinism
 *   (MLSys 2026)", reading notes: "Key observations" 1-4, "Core method /
 *   Target Tests" table, "Recovered Ampere FP16 pipeline", "Experiments and
 *   results").  For one output (i, j) of one step t with C the running FP32
 *   value and P1..P16 the products A[i][16t+k-1]*B[16t+k-1][j]:
 *     - products are exact and unnormalised: sign sa^sb, exponent Ea+Eb,
 *       integer significand ma*mb; subnormal inputs keep exponent emin and
 *       are not renormalised (observations 1 and 3);
 *     - a group sum takes the largest exponent among its non-zero terms,
 *       puts every term on the grid 2^(emax-F) by truncating its magnitude
 *       (round toward zero, observation 3) and adds the integers exactly;
 *     - AMPERE: S1 = C + P1..P8 with F = 23, cut to 24 significant bits
 *       (toward zero, exponent unbounded), then V = S1 + P9..P16 with F = 23
 *       (the two-stage pyramid of observation 2);
 *       HOPPER: V = C + P1..P16 in one group with F = 24 (25-bit width);
 *     - V is written back to FP32 toward zero with gradual underflow;
 *       |V| >= 2^128 becomes +-inf (the BF16 overflow rule of "Experiments
 *       and results", applied to every dtype);
 *     - specials: any NaN, inf*0, or +inf with -inf gives NaN 0x7FC00000,
 *       otherwise an infinite term gives that infinity; a group of only
 *       zero terms gives -0 iff all of them are -0, an exact cancellation
 *       gives +0, an FP32 underflow keeps V's sign;
 *     - the result is the next step's C; after K/16 steps it is D
 *       (observation 4: a MatMul is a deterministic sequence of tiles).
 *   FP8 E4M3 (OCP "FN": no inf, NaN = S.1111.111) exists only with HOPPER.
 *   The optional fingerprint is the XOR of the uint32 patterns of each row
 *   of D ("How AEGIS Turns Training Redundancy into Evidence", section
 *   "Redundancy already exists in the training computation").
 *
 * MEMORY AND LAYOUT
 *   Every pointer is a DEVICE pointer on the current HIP device, owned by
 *   the caller, and aligned to its elements (codes: 2 bytes for FP16 and
 *   BF16; C, D, fingerprint words and step orders: 4 bytes; the audit
 *   report: 8 bytes).
 *   WORKSPACE.  The GEMM entry points stage the operands through a
 *   temporary workspace of operand images, 12 KiB per K-step for each
 *   64-row block of A and each 64-column block of B: all K/16 steps take
 *   12 KiB x (ceil(M/64) + ceil(N/64)) x K/16 bytes (384 MiB at 4096^3).
 *   It is allocated and freed in stream order, around the call's kernels,
 *   from a per-device memory pool that the library creates on first use.
 *   The pool caches nothing: freed workspace returns to the device at the
 *   next synchronisation of the stream, an event or the device, and a
 *   blocking entry point hands it back before it returns, so between
 *   synchronised calls the library holds no device memory
 *   (mma_emulate_workspace_held reports what it holds).  One call takes at
 *   most 1 GiB of workspace.  When the images of all steps do not fit, the
 *   call fills the workspace once per split-K run, or cuts the chain into
 *   runs of steps that restart from the D the previous one wrote (exact:
 *   every step's result is an FP32 value); the results are the same.  If
 *   the allocation fails, or one step's images exceed the cap, the call
 *   stages the operands in LDS instead (same results, slower) and
 *   allocates nothing.  mma_emulate_tiles allocates nothing.  No other
 *   state is kept between calls.
 *   KERNEL CHOICE.  A plain chain runs on a kernel with one lane per
 *   output, which needs no workspace, when an estimate of both kernels'
 *   time says it is the faster (small M * N, or a few rows against a wide
 *   N).  Where that kernel would leave the GPU mostly idle (at most 2048
 *   waves: few outputs, typically with a long K), the chain instead runs
 *   on a kernel that spreads each output over 2 or 4 lanes; its own
 *   pre-pass stages 160 bytes per K-step for each row of A and each column
 *   of B (rows padded to 4 or 8, columns to 16) in the same kind of
 *   workspace, under the same cap and in the same chunks; an audit compare
 *   whose images do not all fit, or a call whose allocation fails, takes
 *   the one-lane kernel.  Shapes over 1,048,560 rows always run on the
 *   tiled kernels, and a plain GEMM over 4,194,240 rows runs in row slices
 *   of that height.  Whichever kernels run, the results are the same.
 *   DIAGNOSTIC OVERRIDES.  Nothing needs to be set in the environment.
 *   Four variables, read on every call and without effect when unset,
 *   force the schedules above so that each can be tested on any shape:
 *   MMAEMU_WORKSPACE_MAX_BYTES (a byte count) replaces the 1 GiB cap;
 *   MMAEMU_NO_WORKSPACE (set to anything) stages every operand of the
 *   tiled kernel in LDS (and leaves the spread kernel none: the one-lane
 *   kernel runs instead);
 *   MMAEMU_NARROW_BLOCKS replaces the kernel estimate by a threshold: the
 *   one-lane-per-output kernels below that many units of 4096 outputs
 *   (M * N), 0 never;
 *   MMAEMU_SPREAD_LANES (0, 2 or 4) decides, where a one-lane-per-output
 *   kernel runs, between the one-lane kernel (0) and the spread kernel
 *   with that many lanes per output.  None of them changes a result.
 *   A  M x K row-major raw codes: uint16 (FP16, BF16) or uint8 (E4M3)
 *   B  K x N row-major raw codes, same type
 *   C  M x N row-major FP32 (read as bit patterns); NULL means all +0.0
 *   D  M x N row-major FP32 bit patterns; D == C (exactly) is allowed
 *   xorsum_out  NULL, or M uint32 words (overwritten, not accumulated; the
 *              words of empty rows, N = 0, are written as 0)
 *   Shapes: M >= 0, N >= 0, K >= 0 with K a multiple of 16.  Empty
 *   operands are allowed (K = 0 gives D = C).
 *
 * ERRORS
 *   Argument errors are reported before anything is enqueued and leave all
 *   buffers untouched.  A failed launch returns MMAEMU_ERR_HIP; the text of
 *   the HIP error is available from mma_emulate_strerror(MMAEMU_ERR_HIP)
 *   on the same thread.  A HIP error that an earlier, unrelated call left
 *   pending in the calling thread (hipGetLastError) is cleared before the
 *   first launch and not reported.  No C++ exception crosses this
 *   interface.
 *
 * DETERMINISM
 *   The same inputs give the same D and xorsum bits on every call, stream
 *   and device.  Each D element is written by exactly one lane (per run of
 *   the split-K schedule, whose runs execute in order); there is no atomic
 *   accumulation of D.
 */
#ifndef MMAEMU_H
#define MMAEMU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* arithmetic models: the architectures the Hawkeye study characterised.
 * LOVELACE computes exactly as AMPERE: the pages report its MMA to have
 * Ampere's structure ("Recovered Ampere FP16 pipeline").  Caveat: they
 * also cite an FP16 product that comes out differently on an L40S and an
 * A100 and keep two simulators ("Problem and motivation", "Experiments and
 * results"), but print nothing that tells the two apart, so no difference
 * is modelled.  FP8 E4M3 is not accepted with LOVELACE. */
enum { MMAEMU_MODEL_AMPERE = 0, MMAEMU_MODEL_HOPPER = 1, MMAEMU_MODEL_LOVELACE = 2 };

/* input formats: FP16, BF16 and FP8 E4M3 ("One-sentence summary") */
enum { MMAEMU_DTYPE_FP16 = 0, MMAEMU_DTYPE_BF16 = 1, MMAEMU_DTYPE_FP8_E4M3 = 2 };

enum {
  MMAEMU_OK = 0,
  MMAEMU_ERR_MODEL = -1,       /* unknown model */
  MMAEMU_ERR_DTYPE = -2,       /* unknown dtype */
  MMAEMU_ERR_UNSUPPORTED = -3, /* E4M3 with a model other than Hopper */
  MMAEMU_ERR_SHAPE = -4,       /* negative size, K not a multiple of 16, overflow */
  MMAEMU_ERR_NULL = -5,        /* a required pointer is NULL */
  MMAEMU_ERR_ALIAS = -6,       /* buffers overlap other than D == C */
  MMAEMU_ERR_HIP = -7,         /* a HIP launch or runtime call failed */
  MMAEMU_ERR_ALIGN = -8,       /* a pointer is not aligned to its elements */
  MMAEMU_ERR_SCRATCH = -9      /* mma_emulate_gemm_noalloc_async: beyond its scratch */
};

/* Emulated GEMM, blocking: enqueued on the null stream of the current
 * device, which is then synchronised.  Arguments as described above. */
int mma_emulate_gemm(int model, int dtype, const void *A, const void *B,
                     const float *C, float *D, int64_t M, int64_t N, int64_t K,
                     uint32_t *xorsum_out);

/* Same contract, enqueued on hip_stream (a hipStream_t; NULL = null
 * stream); returns after enqueue.  The buffers must stay valid until the
 * stream has run the work. */
int mma_emulate_gemm_async(int model, int dtype, const void *A, const void *B,
                           const float *C, float *D, int64_t M, int64_t N,
                           int64_t K, uint32_t *xorsum_out, void *hip_stream);

/* Allocation-free variant of mma_emulate_gemm_async, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors as mma_emulate_gemm_async; it calls no allocator.  Its workspace is
 * a static array of 64 MiB of device memory that the library holds on every
 * GPU it runs on until the process ends, shared by every call on that GPU:
 * calls that overlap on one GPU (on two streams, or from two threads without
 * ordering between them) race on it, so the caller must order them.  Nothing
 * in it needs clearing: each call writes every operand image it reads, and
 * the fingerprint words are cleared on the stream by a kernel.  A chain whose
 * operand images for one K-step exceed the 64 MiB (the tiled kernel with
 * ceil(M/64) + ceil(N/64) > 5461) is rejected with MMAEMU_ERR_SCRATCH before
 * anything is enqueued; a longer chain runs in chunks of as many K-steps as
 * fit, each restarting from the D the previous chunk wrote (the same
 * results).  The workspace overrides of the environment do not apply to
 * it. */
int mma_emulate_gemm_noalloc_async(int model, int dtype, const void *A, const void *B,
                                   const float *C, float *D, int64_t M, int64_t N,
                                   int64_t K, uint32_t *xorsum_out, void *hip_stream);

/* Split-K schedule, an explicit model input.  The pages name split-K (and
 * atomic accumulation) as ways a production library may compose tiles
 * differently from a chain of isolated MMA steps, and leave its
 * characterisation open (Hawkeye notes, "Critical Analysis": the
 * assumption stress test, the missing production path, Future work 4).
 * This entry point fixes one deterministic schedule:
 *   the T = K/16 steps are cut into `splits` runs of T/splits consecutive
 *   steps (splits must divide T; splits = 1 is mma_emulate_gemm_async);
 *   run r chains its steps as mma_emulate_gemm does, starting from C for
 *   r = 0 and from +0 for r > 0, giving the FP32 partial result P_r;
 *   D = (((P_0 + P_1) + P_2) + ... + P_{splits-1}), each addition an
 *   IEEE-754 binary32 addition rounding to nearest, ties to even, with
 *   subnormals kept; a NaN result is the canonical 0x7FC00000.
 * The xorsum fingerprint is taken over the final D.  Arguments, layouts,
 * aliasing (D == C allowed), workspace and errors as for
 * mma_emulate_gemm_async; splits < 1 or not dividing K/16 (or splits != 1
 * with K = 0) is MMAEMU_ERR_SHAPE.  Workspace: when the operand images of
 * all K/16 steps and splits x M x N x 4 bytes of partial results fit under
 * the same cap (and splits <= 65535), the runs are computed side by side
 * and then added in run order; otherwise they run one after another.  The
 * results are the same.  Enqueued on hip_stream; returns after enqueue. */
int mma_emulate_gemm_splitk_async(int model, int dtype, const void *A,
                                  const void *B, const float *C, float *D,
                                  int64_t M, int64_t N, int64_t K, int64_t splits,
                                  uint32_t *xorsum_out, void *hip_stream);

/* Same contract, blocking (null stream, then synchronised). */
int mma_emulate_gemm_splitk(int model, int dtype, const void *A, const void *B,
                            const float *C, float *D, int64_t M, int64_t N,
                            int64_t K, int64_t splits, uint32_t *xorsum_out);

/* K-step order, an explicit model input.  The pages leave the order in
 * which a production library walks K (its tile schedule) to later
 * characterisation (Hawkeye notes, "Critical Analysis": the assumption
 * stress test and the missing production path, Future work 4), and the
 * rounding of every step makes the result depend on it.  This entry point
 * chains the T = K/16 steps in a given order:
 *   C_0 = C;  C_{p+1} = one MMA step of C_p with K-step t = order[p], i.e.
 *   A[:, 16t .. 16t+15] and B[16t .. 16t+15, :];  D = C_T.
 * order: NULL (the forward order 0, 1, .., T-1: mma_emulate_gemm_async), or
 * a DEVICE array of T int32 entries, read-only, which may not overlap D or
 * xorsum_out.  A permutation of 0..T-1 is the intended use; to give every
 * input a defined result, an entry is read as an unsigned 32-bit integer
 * and one at or past T takes step T-1.  Arguments, layouts, workspace,
 * aliasing and errors otherwise as for mma_emulate_gemm_async.  Enqueued
 * on hip_stream; returns after enqueue. */
int mma_emulate_gemm_ordered_async(int model, int dtype, const void *A, const void *B,
                                   const float *C, float *D, int64_t M, int64_t N,
                                   int64_t K, const int32_t *order, uint32_t *xorsum_out,
                                   void *hip_stream);

/* Same contract, blocking (null stream, then synchronised). */
int mma_emulate_gemm_ordered(int model, int dtype, const void *A, const void *B,
                             const float *C, float *D, int64_t M, int64_t N, int64_t K,
                             const int32_t *order, uint32_t *xorsum_out);

/* Audit compare: the auditor's side of the Hawkeye workflow (Hawkeye notes,
 * "Problem and motivation" and "Relation to the verifiable-ML workflow": an
 * auditor who knows only which GPU architecture ran a MatMul recomputes it
 * offline with the characterised arithmetic and checks the provider's
 * published intermediate or final outputs against it; any bit that differs
 * is then wrong execution, not hardware non-determinism).
 * Emulates D = C + A.B exactly as mma_emulate_gemm does
 * and compares every element bit for bit with D_claimed (M x N FP32, read
 * as bit patterns) instead of storing it.  Results, written on the stream:
 *   report        2 uint64 words (device memory, required):
 *                   report[0] = number of elements whose bits differ,
 *                   report[1] = row-major index i*N + j of the first
 *                               (smallest-index) differing element, or
 *                               UINT64_MAX when none differs;
 *   row_diff_out  NULL, or M uint32 words (overwritten): word i is the XOR
 *                 over j of (emulated ^ claimed) bits of row i.  A non-zero
 *                 word proves that row differs; differences can cancel in
 *                 the XOR, so a zero word proves nothing (report[0] is
 *                 exact).
 * A, B, C and D_claimed are read-only and may overlap one another; report
 * and row_diff_out may overlap nothing.  Shapes, NULL C and errors as for
 * mma_emulate_gemm; D_claimed may be NULL only when M*N == 0.  Enqueued on
 * hip_stream; returns after enqueue. */
int mma_verify_gemm_async(int model, int dtype, const void *A, const void *B,
                          const float *C, const float *D_claimed, int64_t M,
                          int64_t N, int64_t K, uint64_t *report,
                          uint32_t *row_diff_out, void *hip_stream);

/* Same contract, blocking: enqueued on the null stream of the current
 * device, which is then synchronised. */
int mma_verify_gemm(int model, int dtype, const void *A, const void *B,
                    const float *C, const float *D_claimed, int64_t M, int64_t N,
                    int64_t K, uint64_t *report, uint32_t *row_diff_out);

/* ntiles independent 16x16x16 MMA steps (the unit the Hawkeye study audits,
 * "Key observation 1"): A, B are [ntiles][16][16] row-major codes, C, D are
 * [ntiles][16][16] FP32 (C may be NULL, D may equal C); xorsum_out is NULL
 * or ntiles words, each the XOR of its tile's 256 D words.  Enqueued on
 * hip_stream; returns after enqueue. */
int mma_emulate_tiles(int model, int dtype, const void *A, const void *B,
                      const float *C, float *D, int64_t ntiles,
                      uint32_t *xorsum_out, void *hip_stream);

/* Bytes of device memory that the workspace pool of HIP device `device`
 * holds right now (0 before the pool exists), written to *bytes_out (host
 * memory).  After a blocking entry point returns, and after any
 * synchronisation that follows the asynchronous ones, it is 0.  Errors:
 * MMAEMU_ERR_NULL for a NULL bytes_out, MMAEMU_ERR_HIP for a device that
 * does not exist. */
int mma_emulate_workspace_held(int device, uint64_t *bytes_out);

/* Text for a return code (thread-local for MMAEMU_ERR_HIP: names the last
 * HIP error seen on this thread).  Never NULL. */
const char *mma_emulate_strerror(int code);

/* Revision of the arithmetic rules above; bumped whenever a rule changes. */
int mma_emulate_spec_version(void);

#ifdef __cplusplus
}
#endif
#endif
