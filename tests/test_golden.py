"""The oracle reproduces its recorded outputs on tiny seeded inputs (a
regression record; the oracle's correctness is pinned in test_oracle_pins)."""
import os
import sys

import numpy as np
import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, HERE)
import make_golden  # noqa: E402


@pytest.mark.parametrize("name", sorted(make_golden.TINY))
def test_golden(name):
    with open(os.path.join(HERE, f"{name}_tiny_seed0.txt")) as f:
        vals = [float.fromhex(l.strip()) for l in f if l.strip() and not l.startswith("#")]
    y = make_golden.golden_output(name, make_golden.TINY[name])
    # BLAS kernels differ between hosts, so allow last-bit differences
    np.testing.assert_allclose(y.reshape(-1), np.array(vals), rtol=1e-13, atol=1e-15)
