"""The oracle against what the definitions and mathematics fix (CPU only).

Each check lives in tests/pins.py; see there for what it recomputes and
how.  Together they pin the neighbour count, the core flag, the merge, the
border rule and the labels of the brute-force oracle to hand-worked cases,
exact rational arithmetic, a breadth-first DBSCAN, scipy and scikit-learn.
"""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, check):
    check(orc)
