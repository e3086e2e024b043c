"""The oracle-digest cache (tests/golden/oracle_digests.json) is keyed by
what made it: every entry's input digest must be reproduced by today's
seeded generator, and its oracle-source digest must be today's oracle's.  A
stale entry then fails here, on the CPU, instead of passing for the current
oracle in the GPU tests."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_digests as MD  # noqa: E402


def test_every_entry_is_keyed_to_the_current_oracle_and_inputs():
    data = json.load(open(MD.OUT))
    workloads = MD.workloads()
    assert set(data) == set(workloads)
    current = MD.oracle_source_sha256()
    for name, (kind, model, dt, gen) in workloads.items():
        e = data[name]
        assert e["oracle_source_sha256"] == current, (
            f"{name}: made by another revision of the oracle; rerun tests/golden/make_digests.py")
        A, B, C = gen()
        assert e["inputs_sha256"] == MD.inputs_sha256(A, B, C), (
            f"{name}: the seeded generator no longer gives these inputs")
        assert (e["model"], e["dtype"]) == (model, dt)
