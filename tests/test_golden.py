"""The stored oracle fixture for the tiny workload must still reproduce."""

import json
import os

import numpy as np

from tests.golden.make_golden import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_fixture_reproduces():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        stored = json.load(f)
    now = build()
    assert now["argmax"] == stored["argmax"]
    assert now["accept_len"] == stored["accept_len"]
    assert now["draft"] == stored["draft"]
    np.testing.assert_allclose(np.array(now["y_sample"], dtype=float),
                               np.array(stored["y_sample"], dtype=float), rtol=1e-13)
    np.testing.assert_allclose(np.array(now["y_row_sums"], dtype=float),
                               np.array(stored["y_row_sums"], dtype=float), rtol=1e-12)
    # the first three drafts were forced to the argmax, so at least 3 accept
    assert stored["accept_len"][0] >= 3
