"""Consistency of the stored oracle outputs (tests/golden/pass_cfg*.npz)
written by tests/golden/make_golden.py: the stored top logits are sorted,
each drafted token is the arg-max of its position's logits, the sampled
logits never exceed the top one, and the confidences are probabilities."""
import glob
import os

import numpy as np
import pytest

FILES = sorted(glob.glob(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pass_cfg*.npz")))


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(f) for f in FILES])
def test_golden_internally_consistent(path):
    g = np.load(path)
    top_val, top_idx = g["top_val"], g["top_idx"]
    assert (np.diff(top_val, axis=2) <= 0).all()
    np.testing.assert_array_equal(g["tokens"], top_idx[:, :, 0])
    assert (g["smp_val"] <= top_val[:, :, :1] + 0.0).all()
    assert ((g["conf"] > 0) & (g["conf"] < 1)).all()
    assert np.isfinite(g["hidden_val"]).all()
