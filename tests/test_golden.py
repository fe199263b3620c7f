"""The stored oracle outputs for the tiny case still match the oracle exactly."""
import json
import os

import numpy as np

from tests.golden.make_golden import tiny_oracle


def test_tiny_case_fixture_matches_oracle():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_case_oracle.json")
    with open(path) as f:
        ref = json.load(f)
    o, S = tiny_oracle()
    assert np.array_equal(o, np.array(ref["o"], dtype=np.float64))
    assert np.array_equal(S, np.array(ref["S_T"], dtype=np.float64))
