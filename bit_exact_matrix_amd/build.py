"""Build libmmaemu.so in-tree with hipcc for gfx950.

``python -m bit_exact_matrix_amd.build`` builds the library;
``python -m bit_exact_matrix_amd.build probe`` builds, in addition, the VALU
issue-rate probe that ``bench.py --valu-peak`` loads (a measurement aid,
not part of the library).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmmaemu.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no packed-FP32 instruction selection anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # all packed 16-bit arithmetic in the kernels is explicit; the SLP
    # vectoriser only pairs scalar epilogue ops at a net cost
    "-fno-slp-vectorize",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


PROBE_SRC = os.path.join(HERE, "probe", "valu_rate.hip")
PROBE_OUT = os.path.join(HERE, "probe", "libvalurate.so")


def _hipcc(src: str, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


def build(out: str = OUT, verbose: bool = False) -> str:
    """libmmaemu.so, the library."""
    return _hipcc(os.path.join(CSRC, "mmaemu.hip"), out, verbose)


def build_probe(verbose: bool = False) -> str:
    """libvalurate.so, the VALU issue-rate probe of bench.py --valu-peak."""
    return _hipcc(PROBE_SRC, PROBE_OUT, verbose)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "probe":
        print(build_probe(verbose=True))
    print(build(verbose=True))
