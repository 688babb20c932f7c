"""Regression of the oracle against fixtures written by tests/golden/make_golden.py."""
import json
import os

import numpy as np
import pytest

from tests.golden import make_golden as G

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("case", G.CASES, ids=lambda c: c["name"])
def test_oracle_matches_frozen_fixture(case):
    with open(os.path.join(HERE, case["name"] + ".json")) as f:
        rec = json.load(f)
    got = G.compute(case)
    for key, want in rec["values"].items():
        np.testing.assert_allclose(np.array(got[key]), np.array(want), rtol=1e-12, atol=1e-13,
                                   err_msg=key)
