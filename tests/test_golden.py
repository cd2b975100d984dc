"""The oracle still reproduces the stored fixtures of tests/golden/small_cases.json.

The fixtures were written by tests/golden/make_golden.py from the oracle alone
(the pages print no numeric outputs); this guards the oracle against silent
drift.  The GPU parity tests reuse the same cases.
"""
import json
import os

import numpy as np
import pytest

import oracle

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "small_cases.json")
CASES = json.load(open(PATH))


@pytest.mark.parametrize("name", sorted(CASES))
def test_oracle_matches_golden(name):
    c = CASES[name]
    x, y = np.float32(c["x"]), np.float32(c["y"])
    b, g = np.float32(c["b"]), np.float32(c["g"])
    a, n = oracle.gauss_sum(x, y, b, c["sigma"])
    np.testing.assert_allclose(a, c["sum"], rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(n, c["sum_norm"], rtol=1e-14)
    np.testing.assert_allclose(oracle.gauss_lse(x, y, b, c["sigma"]), c["lse"], rtol=1e-14)
    G, nu = oracle.gauss_grad_x(x, y, b, g, c["sigma"])
    np.testing.assert_allclose(G, c["grad_x"], rtol=1e-13, atol=1e-14 * max(1.0, np.max(nu)))
    Gy, nuy = oracle.gauss_grad_y(x, y, b, g, c["sigma"])
    np.testing.assert_allclose(Gy, c["grad_y"], rtol=1e-13, atol=1e-14 * max(1.0, np.max(nuy)))
    Gb, nub = oracle.gauss_grad_b(x, y, g, c["sigma"])
    np.testing.assert_allclose(Gb, c["grad_b"], rtol=1e-13, atol=1e-14 * max(1.0, np.max(nub)))
    kd, ki = oracle.kmin(x, y, c["K"])
    assert ki.tolist() == c["kmin_idx"]
    np.testing.assert_allclose(kd, c["kmin_d"], rtol=1e-15)
