"""The oracle still reproduces its stored output for the tiny workload."""
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_workload_regression():
    want = np.loadtxt(os.path.join(HERE, "cfg_tiny_seed0.txt"))
    got = compute().ravel()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
