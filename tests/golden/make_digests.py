"""Write oracle_digests.json: SHA-256 digests of the CPU oracle's outputs on
the seeded workloads, so GPU tests can check full-size results bit for bit
without re-running the oracle for minutes.  Calls only oracle/ and the seeded
input generators.  Run:  python tests/golden/make_digests.py [names...]

Each entry is keyed by what determines it: the digest of its input bits
(A, B, C from the seeded generator) and the digest of the oracle's sources.
tests/test_oracle_digests.py checks both against the current tree, so that
a cache made by another oracle or from other inputs cannot pass for this
one's.
"""
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from bit_exact_matrix_amd import inputs as I  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digests.json")


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


ORACLE_SOURCES = ("oracle/mma_oracle.c", "oracle/mma_oracle.h", "oracle/__init__.py")


def oracle_source_sha256():
    h = hashlib.sha256()
    for rel in ORACLE_SOURCES:
        h.update(rel.encode() + b"\0" + open(os.path.join(ROOT, rel), "rb").read() + b"\0")
    return h.hexdigest()


def inputs_sha256(A, B, C):
    h = hashlib.sha256()
    for a in (A, B, C):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def workloads():
    """name -> (kind, model, dtype, generator) for the five seeded configs
    (and the 4096^3 FP16 Ampere GEMM under the 4-run split-K schedule and
    with its 256 K-steps in reversed order)."""
    return {
        "tiles_fp16_1k_ampere": ("tiles", "ampere", "fp16", lambda: I.tiles_normal(1001, 1000)),
        "tiles_mixed_100k_fp16_ampere": ("tiles", "ampere", "fp16",
                                         lambda: I.tiles_mixed(2001, 100000, I.FP16)),
        "tiles_mixed_100k_fp16_hopper": ("tiles", "hopper", "fp16",
                                         lambda: I.tiles_mixed(2001, 100000, I.FP16)),
        "tiles_mixed_100k_bf16_ampere": ("tiles", "ampere", "bf16",
                                         lambda: I.tiles_mixed(2002, 100000, I.BF16)),
        "tiles_mixed_100k_bf16_hopper": ("tiles", "hopper", "bf16",
                                         lambda: I.tiles_mixed(2002, 100000, I.BF16)),
        "gemm_4096_fp16_ampere": ("gemm", "ampere", "fp16",
                                  lambda: I.gemm_normal(3001, 4096, 4096, 4096)),
        "gemm_4096_bf16_hopper": ("gemm", "hopper", "bf16",
                                  lambda: I.gemm_wide_bf16(4001, 4096, 4096, 4096)),
        "gemm_4096_e4m3_hopper": ("gemm", "hopper", "e4m3",
                                  lambda: I.gemm_e4m3(5001, 4096, 4096, 4096)),
        "gemm_4096_fp16_ampere_splitk4": ("splitk4", "ampere", "fp16",
                                          lambda: I.gemm_normal(3001, 4096, 4096, 4096)),
        "gemm_4096_fp16_ampere_reversed": ("reversed", "ampere", "fp16",
                                           lambda: I.gemm_normal(3001, 4096, 4096, 4096)),
    }


def main(names):
    oracle.build(force=False)
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name, (kind, model, dt, gen) in workloads().items():
        if names and name not in names:
            continue
        A, B, C = gen()
        t = time.time()
        if kind == "tiles":
            D, x = oracle.tiles(model, dt, A, B, C)
        elif kind == "splitk4":
            D, x = oracle.gemm_splitk(model, dt, A, B, C, 4)
        elif kind == "reversed":
            T = A.shape[1] // 16
            D, x = oracle.gemm_ordered(model, dt, A, B, C, np.arange(T - 1, -1, -1, dtype=np.int32))
        else:
            D, x = oracle.gemm(model, dt, A, B, C)
        dt_s = time.time() - t
        data[name] = {"model": model, "dtype": dt, "shape": list(D.shape),
                      "D_sha256": sha(D), "xorsum_sha256": sha(x),
                      "xorsum_head": [f"{int(v):#010x}" for v in x[:4]],
                      "D_head": [f"{int(v):#010x}" for v in D.reshape(-1)[:4]],
                      "n_inf": int(((D & 0x7FFFFFFF) == 0x7F800000).sum()),
                      "n_nan": int(((D & 0x7FFFFFFF) > 0x7F800000).sum()),
                      "oracle_seconds": round(dt_s, 1), "oracle_threads": oracle.num_cpus(),
                      "inputs_sha256": inputs_sha256(A, B, C),
                      "oracle_source_sha256": oracle_source_sha256()}
        print(name, data[name], flush=True)
        json.dump(data, open(OUT, "w"), indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
