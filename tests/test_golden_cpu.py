"""The oracle's stored digests of the five named workloads are complete and
still describe the generator's output (no GPU needed).  The GPU parity
tests compare against these digests and fail if an entry is missing."""
import json
import os

import pytest

import pins
from all_pairs_distance_amd import datagen

GOLDEN_WORKLOADS = os.path.join(pins.GOLDEN, "workloads.json")


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_workload_digests_present_and_current(key):
    g = json.load(open(GOLDEN_WORKLOADS)).get(str(key))
    assert g is not None
    for field in ("labels_sha256", "counts_sha256", "points_sha256", "n_core"):
        assert field in g
    x, eps, m, w = datagen.make_workload(key)
    assert g["points_sha256"] == datagen.sha256_points(x), w.name
    assert "expanded" in g and "labels_sha256" in g["expanded"]
