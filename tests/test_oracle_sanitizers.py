"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc; any report aborts) and driven through its whole C interface in a
child process: shifts past the word width, signed overflow and
out-of-bounds accesses in the arithmetic or the threaded row split would
stop it.  Host code only."""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    import numpy as np
    import oracle
    from bit_exact_matrix_amd import inputs as I
    lib = oracle.Library({so!r}).lib
    rng = np.random.default_rng(3)
    from test_oracle_pins import _random_dot_inputs
    for model, dt in ((0, 0), (1, 0), (0, 1), (1, 1), (1, 2)):
        for adv in (False, True):
            a, b, c = _random_dot_inputs(rng, dt, 3000, adv)
            oracle.dots(model, dt, a, b, c, lib=lib)
    for model, dt, dti in (("ampere", "fp16", I.FP16), ("hopper", "bf16", I.BF16),
                           ("hopper", "e4m3", I.E4M3), ("lovelace", "bf16", I.BF16)):
        for mode in ("wide", "coarse", "tiny"):
            A, B, C = I.gemm_adversarial(11, 37, 29, 64, dti, mode)
            oracle.gemm(model, dt, A, B, C, nthreads=4, lib=lib)
            oracle.gemm_rows(model, dt, A, B, C, 3, 20, nthreads=3, lib=lib)
            oracle.gemm_splitk(model, dt, A, B, C, 2, nthreads=2, lib=lib)
        A, B, C = I.gemm_specials(12, 21, 19, 48, dti)
        oracle.gemm(model, dt, A, B, C, nthreads=2, lib=lib)
    A, B, C = I.tiles_mixed(13, 400, I.BF16)
    oracle.tiles("hopper", "bf16", A, B, C, nthreads=3, lib=lib)
    print("sanitized oracle: ok")
""")


def _run_sanitized(tmp_path, source_text):
    src = tmp_path / "oracle_san.c"
    src.write_text(source_text)
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c99", "-D_DEFAULT_SOURCE", "-O1", "-g", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-pthread", "-I", os.path.dirname(oracle.SRC),
                    str(src), "-o", so], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no shared AddressSanitizer runtime")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]))
    return subprocess.run([sys.executable, "-c", DRIVER.format(root=ROOT, so=so)], env=env,
                          capture_output=True, text=True, timeout=600)


def test_oracle_under_asan_and_ubsan(tmp_path):
    r = _run_sanitized(tmp_path, open(oracle.SRC).read())
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert "sanitized oracle: ok" in r.stdout


def test_the_sanitizers_are_live(tmp_path):
    """Without the guard on the alignment distance, shifting by 64 or more is
    undefined behaviour; the same driver must stop on it."""
    text = open(oracle.SRC).read()
    guard = "  if (d >= 63) return 0;\n  return mag >> d;"
    assert guard in text
    r = _run_sanitized(tmp_path, text.replace(guard, "  return mag >> d;"))
    assert r.returncode != 0
    assert "shift exponent" in r.stderr
