"""Regression guard: the oracle still reproduces tests/golden/tiny_conv_sample.json
(written by tests/golden/make_golden.py, which calls only the oracle)."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_sample_unchanged():
    with open(os.path.join(HERE, "golden", "tiny_conv_sample.json")) as f:
        ref = json.load(f)
    got = compute()
    assert got["n_edges"] == ref["n_edges"] == 1024
    for k in ("m", "dx", "dw", "dY"):
        np.testing.assert_allclose(np.array(got[k]), np.array(ref[k]), rtol=1e-12, atol=1e-12)
