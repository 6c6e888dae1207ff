"""The oracle still reproduces its stored regression fixture (CPU only)."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_stored_fixture():
    with open(os.path.join(HERE, "oracle_small.json")) as f:
        want = json.load(f)
    got = compute()
    for key in ("idx", "counts", "offsets", "dest", "src"):
        assert got[key] == want[key], key
    for key in ("w", "y", "dx", "dwr", "dw1_sum", "dw2_sum"):
        np.testing.assert_allclose(got[key], want[key], rtol=1e-12, atol=1e-14)
