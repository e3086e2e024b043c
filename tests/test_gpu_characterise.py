"""The characterisation harness pointed at the GPU emulator: every probe's
dot products run through mma_emulate_tiles, bit-identical to the oracle's,
and the recovered model table equals the pages' Target Tests results."""
import json
import os

import numpy as np
import pytest

from bit_exact_matrix_amd import characterise as ch
from test_gpu_parity import say, torch_dev  # noqa: F401

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = json.load(open(os.path.join(HERE, "golden", "target_tests.json")))["models"]
COMBOS = [("ampere", "fp16"), ("hopper", "fp16"), ("ampere", "bf16"), ("hopper", "bf16"),
          ("hopper", "e4m3"), ("lovelace", "fp16")]


@pytest.mark.parametrize("model,dtype", COMBOS)
def test_gpu_characterisation(torch_dev, orc, model, dtype):
    gpu = ch.gpu_dots(model, dtype)
    calls = []

    def checked(a, b, c):
        d = gpu(a, b, c)
        want = orc.dots(model, dtype, a, b, c)
        bad = np.nonzero(d != want)[0]
        assert bad.size == 0, (f"{model}/{dtype}: {bad.size} of {len(c)} probe dot products "
                               f"differ from the oracle, first row {bad[0]}")
        calls.append(len(c))
        return d

    say("characterise", model, dtype)
    got = ch.characterise(checked, dtype)
    for key, want in TABLE[model].items():
        assert got[key] == want, (model, dtype, key, got[key])
    assert sum(calls) > 262000   # the full neutral-subgroup enumeration ran
