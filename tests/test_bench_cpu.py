"""bench.py host logic (no GPU): refusal of more than one GPU and the
consistency of its workload tables with the stored oracle digests."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_every_workload_has_a_stored_digest_and_known_generator():
    from bit_exact_matrix_amd import inputs
    dig = json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))
    assert bench.DEFAULT_WORKLOAD in bench.WORKLOADS
    for name, (model, mid, dt, did, (gen, seed), data, pages_s) in bench.WORKLOADS.items():
        rec = dig[bench.DIGEST_KEY[name]]
        assert rec["model"] == model and rec["dtype"] == dt
        assert rec["shape"] == [bench.M, bench.N]
        assert callable(getattr(inputs, gen))
        assert model in bench.ALG_SLOTS_PER_MAC and pages_s > 0


def test_default_metric_names_the_fp16_ampere_gemm():
    model, _, dt, _, _, _, _ = bench.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (f"bit-exact emulated MACs/s, 4096³ {dt.upper()} {model.capitalize()} model; "
            f"% of VALU peak") == "bit-exact emulated MACs/s, 4096³ FP16 Ampere model; % of VALU peak"


def test_every_tile_workload_has_a_stored_digest():
    from bit_exact_matrix_amd import inputs
    dig = json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))
    for name, (model, mid, dt, did, (gen, gargs), data, key) in bench.TILE_WORKLOADS.items():
        rec = dig[key]
        assert rec["model"] == model and rec["dtype"] == dt
        assert rec["shape"][0] == gargs[1]
        assert callable(getattr(inputs, gen))


def test_shape_mode_rejects_bad_shapes_before_touching_a_gpu():
    for shape, mma in (("10x10x15", "ampere/fp16"), ("0x16x16", "ampere/fp16"),
                       ("16x16", "ampere/fp16"), ("16x16x16", "volta/fp16"),
                       ("16x16x16", "ampere/fp32"), ("16x16x48", "ampere/fp16 --splits 2")):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--shape", shape,
                            "--mma", *mma.split()], capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, (shape, mma, r.stderr[-300:])
        assert "--shape takes MxNxK" in r.stderr
        assert r.stdout == ""
