"""The oracle has not drifted from the stored tiny-workload fixture (written by
tests/golden/make_golden.py, which calls only the oracle)."""

import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_stored_fixture():
    with open(os.path.join(HERE, "golden", "tiny_fp32_oracle.json")) as f:
        ref = json.load(f)
    now = compute()
    for key in ("o", "S_row0", "S_sum"):
        np.testing.assert_allclose(np.array(now[key]), np.array(ref[key]), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(now["o_abs_sum"], ref["o_abs_sum"], rtol=1e-12)
