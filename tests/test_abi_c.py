"""The C ABI from C: include/mmaemu.h compiles as strict C99, a C program
links against libmmaemu.so, and every entry point answers its argument
errors with the documented codes before any HIP call (no GPU needed)."""
import os
import subprocess

import pytest

import bit_exact_matrix_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mmaemu.h"

#define EXPECT(call, code) do { int rc_ = (call); if (rc_ != (code)) { \
  printf("FAIL %s: %d, expected %d\n", #call, rc_, (code)); return 1; } } while (0)

int main(void) {
  /* fake device addresses: validation must reject every call before use */
  const void *A = (const void *)0x10000000, *B = (const void *)0x20000000;
  const float *C = (const float *)0x30000000;
  float *D = (float *)0x40000000;
  uint32_t *X = (uint32_t *)0x50000000;
  uint64_t *R = (uint64_t *)0x60000000;
  const int32_t *O = (const int32_t *)0x70000000;
  EXPECT(mma_emulate_gemm(9, MMAEMU_DTYPE_FP16, A, B, C, D, 32, 32, 32, X), MMAEMU_ERR_MODEL);
  EXPECT(mma_emulate_gemm_async(MMAEMU_MODEL_AMPERE, 7, A, B, C, D, 32, 32, 32, X, NULL),
         MMAEMU_ERR_DTYPE);
  EXPECT(mma_emulate_gemm_splitk(MMAEMU_MODEL_AMPERE, MMAEMU_DTYPE_FP8_E4M3, A, B, C, D, 32, 32,
                                 32, 1, X), MMAEMU_ERR_UNSUPPORTED);
  EXPECT(mma_emulate_gemm_splitk_async(MMAEMU_MODEL_HOPPER, MMAEMU_DTYPE_BF16, A, B, C, D, 32,
                                       32, 48, 2, X, NULL), MMAEMU_ERR_SHAPE);
  EXPECT(mma_verify_gemm(MMAEMU_MODEL_HOPPER, MMAEMU_DTYPE_FP16, A, B, C, D, 32, 32, 32, NULL,
                         X), MMAEMU_ERR_NULL);
  EXPECT(mma_verify_gemm_async(MMAEMU_MODEL_LOVELACE, MMAEMU_DTYPE_BF16, A, B, C, D, 32, 32, 32,
                               R, (uint32_t *)R, NULL), MMAEMU_ERR_ALIAS);
  EXPECT(mma_emulate_tiles(MMAEMU_MODEL_AMPERE, MMAEMU_DTYPE_FP16, A, B, C, D, -1, X, NULL),
         MMAEMU_ERR_SHAPE);
  EXPECT(mma_emulate_tiles(MMAEMU_MODEL_HOPPER, MMAEMU_DTYPE_FP16, A, B, C, D, 0, X, NULL),
         MMAEMU_OK);
  /* misaligned pointers: codes off their 2-byte elements, atomically
     updated words off their natural alignment */
  EXPECT(mma_emulate_gemm(MMAEMU_MODEL_AMPERE, MMAEMU_DTYPE_FP16, (const char *)A + 1, B, C,
                          D, 32, 32, 32, X), MMAEMU_ERR_ALIGN);
  EXPECT(mma_emulate_gemm_async(MMAEMU_MODEL_HOPPER, MMAEMU_DTYPE_BF16, A, B, C, D, 32, 32, 32,
                                (uint32_t *)((char *)X + 2), NULL), MMAEMU_ERR_ALIGN);
  EXPECT(mma_verify_gemm(MMAEMU_MODEL_HOPPER, MMAEMU_DTYPE_FP16, A, B, C, D, 32, 32, 32,
                         (uint64_t *)((char *)R + 4), X), MMAEMU_ERR_ALIGN);
  EXPECT(mma_emulate_tiles(MMAEMU_MODEL_AMPERE, MMAEMU_DTYPE_BF16, A, B, C,
                           (float *)((char *)D + 2), 4, X, NULL), MMAEMU_ERR_ALIGN);
  EXPECT(mma_emulate_gemm_ordered(MMAEMU_MODEL_AMPERE, MMAEMU_DTYPE_FP16, A, B, C, D, 32, 32,
                                  32, (const int32_t *)((const char *)O + 2), X),
         MMAEMU_ERR_ALIGN);
  EXPECT(mma_emulate_gemm_ordered_async(MMAEMU_MODEL_HOPPER, MMAEMU_DTYPE_FP8_E4M3, A, B, C,
                                        D, 32, 32, 32, (const int32_t *)D, X, NULL),
         MMAEMU_ERR_ALIAS);
  {
    uint64_t held = 1;
    EXPECT(mma_emulate_workspace_held(0, NULL), MMAEMU_ERR_NULL);
    EXPECT(mma_emulate_workspace_held(-1, &held), MMAEMU_ERR_HIP);
  }
  if (mma_emulate_spec_version() < 1) return 1;
  if (strcmp(mma_emulate_strerror(MMAEMU_OK), "ok") != 0) return 1;
  printf("c abi: ok\n");
  return 0;
}
"""


def test_header_compiles_as_c99_and_a_c_program_links(tmp_path):
    lib = mm.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libmmaemu.so is not built")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = str(tmp_path / "abi")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", exe,
                    "-L", os.path.dirname(lib), "-lmmaemu",
                    "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi: ok" in r.stdout
