/*
 * mma_oracle.h -- plain CPU oracle for the bit-exact tile-MMA emulation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no source with the HIP
 * library: the two meet only at the bit level (same input codes in, same
 * FP32 bit patterns out).
 *
 * Arithmetic followed (sources: "Hawkeye: Reproducing GPU-Level
 * Non-Determinism (MLSys 2026)" reading notes -- sections "Key observations"
 * (observations 1-4), "Core method / Target Tests" table, "Recovered Ampere
 * FP16 pipeline", "Experiments and results"; "How AEGIS Turns Training
 * Redundancy into Evidence" for the xorsum fingerprint).  The full list of
 * rules, and the readings taken where the pages are silent, is in the
 * comments of mma_oracle.c.
 *
 * All pointers are HOST pointers.  Layouts:
 *   A  M x K row-major raw codes (uint16 for FP16/BF16, uint8 for E4M3)
 *   B  K x N row-major raw codes
 *   C  M x N row-major FP32 bit patterns (NULL = all +0.0)
 *   D  M x N row-major FP32 bit patterns (may equal C)
 *   xorsum_out  NULL or M words: XOR over j of D[i][j]
 * K must be a multiple of 16 (K/16 chained 16x16x16 steps); M, N >= 0.
 * Return 0 on success, negative on a bad argument (nothing written).
 */
#ifndef MMA_ORACLE_H
#define MMA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ORC_LOVELACE follows the Ampere rules (R12 in mma_oracle.c) */
enum { ORC_AMPERE = 0, ORC_HOPPER = 1, ORC_LOVELACE = 2 };
enum { ORC_FP16 = 0, ORC_BF16 = 1, ORC_E4M3 = 2 };

/* Full GEMM, rows distributed over nthreads host threads (0 = all cores). */
int mma_oracle_gemm(int model, int dtype, const void *A, const void *B,
                    const uint32_t *C, uint32_t *D, int64_t M, int64_t N,
                    int64_t K, uint32_t *xorsum_out, int nthreads);

/* Rows [row_begin, row_end) of the same GEMM.  A, B, C are the full
 * operands; D_rows and xorsum_rows receive (row_end-row_begin) rows only. */
int mma_oracle_gemm_rows(int model, int dtype, const void *A, const void *B,
                         const uint32_t *C, uint32_t *D_rows, int64_t M,
                         int64_t N, int64_t K, int64_t row_begin,
                         int64_t row_end, uint32_t *xorsum_rows, int nthreads);

/* ntiles independent 16x16x16 MMAs: A, B, C, D are [ntiles][16][16]
 * row-major; xorsum_out is NULL or ntiles words (XOR of the tile's D). */
int mma_oracle_tiles(int model, int dtype, const void *A, const void *B,
                     const uint32_t *C, uint32_t *D, int64_t ntiles,
                     uint32_t *xorsum_out, int nthreads);

/* n single outputs of one MMA step: d[r] = step(c[r], a[r][0..15],
 * b[r][0..15]), a and b holding raw codes (uint16 / uint8). */
int mma_oracle_dots(int model, int dtype, const void *a, const void *b,
                    const uint32_t *c, uint32_t *d, int64_t n);

int mma_oracle_num_cpus(void);

#ifdef __cplusplus
}
#endif
#endif
