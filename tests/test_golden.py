"""The oracle still reproduces its stored tiny-case outputs (regression pin, CPU only)."""
import json
import os

import numpy as np

from tests.golden import make_golden


def test_oracle_matches_stored_tiny_case():
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    with open(path) as f:
        stored = json.load(f)["values"]
    now = make_golden.case()
    assert set(stored) == set(now)
    for k in stored:
        a, b = np.asarray(stored[k], dtype=float), np.asarray(now[k], dtype=float)
        assert a.shape == b.shape, k
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14, equal_nan=True), k
