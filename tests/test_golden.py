"""The oracle still reproduces its stored golden fixture (regression lock)."""
import json
import os

import numpy as np

from tests.golden import make_golden


def test_oracle_matches_stored_fixture():
    with open(make_golden.OUT) as f:
        doc = json.load(f)
    o1, o2, l2 = make_golden.expected()
    np.testing.assert_allclose(o1.ravel(), doc["phase1_out"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(o2.ravel(), doc["phase2_out"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2.ravel(), doc["phase2_lse"], rtol=0, atol=1e-13)
