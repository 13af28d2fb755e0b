"""The stored tiny-workload outputs still match the oracle (CPU only).

The fixture was written by ``tests/golden/make_tiny_fixture.py``, which calls
only the oracle; this test catches any later change to the oracle's arithmetic.
"""
import os

import numpy as np

from golden.make_tiny_fixture import OUT, run_oracle


def test_tiny_fixture_matches_oracle():
    stored = np.loadtxt(OUT, comments="#")
    o, S = run_oracle()
    fresh = np.concatenate([o.ravel(), S.ravel()])
    assert stored.shape == fresh.shape
    assert np.max(np.abs(stored - fresh)) <= 1e-15 * np.max(np.abs(stored))


def test_tiny_fixture_is_sane():
    stored = np.loadtxt(OUT, comments="#")
    assert np.all(np.isfinite(stored))
    o = stored[:16 * 4 * 16].reshape(16, 4, 16)
    # with q scaled by 1/sqrt(16) and a BF16-rounded N(0, 0.1) state, outputs stay O(1)
    assert 1e-3 < np.max(np.abs(o)) < 10
