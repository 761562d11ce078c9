"""Parity of the hoisted-norm distance form (DBSCAN_FLAG_EXPANDED) with the
oracle's form of it (Wang et al. Sec. IV-B2: T + P - sum 2 x_k y_k, every
step a binary32 operation in a fixed order).

Counts, labels and graphs must be bit-identical to the oracle run with
form="expanded".  Many inputs sit far from the origin, where the two forms
decide many pairs differently and the screen hands most pairs near the
radius to the exact path; the tests check that such disagreements are
present, so they cannot pass on the direct form by accident.
"""
import hashlib
import json
import os

import numpy as np
import pytest

import pins
from all_pairs_distance_amd import datagen
from test_gpu_parity import _screen_cases, assert_same, gpu_fit
from test_gpu_graph import assert_same_graph, gpu_graph

pytestmark = pytest.mark.gpu

EXP = 0x20
# with the edge list, with the tile merge, with the schedule walked backwards
MODES = [(EXP, "edges"), (EXP | 0x2, "tiles"), (EXP | 0x10, "reverse"),
         (EXP | 0x8, "with_screen_flag")]


@pytest.fixture(scope="module")
def apd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import all_pairs_distance_amd
    return all_pairs_distance_amd


@pytest.mark.parametrize("flags,mode", MODES, ids=[m for _, m in MODES])
def test_expanded_small_and_far_sets(apd, orc, flags, mode):
    disagree = 0
    cases = pins.small_cases(seed=131, count=50) + pins.far_cases(seed=137, count=40)
    # wide points (the matrix-core pass), near and far from the origin
    for d, off in ((33, 0.0), (48, 50.0), (64, 10.0)):
        x = datagen.gaussian_blobs(3000, d, seed=900 + d, n_blobs=6, sigma=0.04,
                                   noise_frac=0.1)
        cases.append(((x + np.float32(off)).astype(np.float32),
                      0.05 * float(np.sqrt(d)), 4))
    for t, (x, eps, m) in enumerate(cases):
        want_l, want_c, _ = orc.fit(x, eps, m, form="expanded")
        lab, cnt, info = gpu_fit(apd, x, eps, m, flags=flags)
        assert_same(lab, cnt, want_l, want_c, f"case {t} n={x.shape} eps={eps} m={m}")
        if x.shape[0] > 0 and info["n_core"] > 0:
            assert info["merge_mode"] == (2 if flags & 2 else 1)
        disagree += int(np.sum(orc.fit(x, eps, m)[1] != want_c))
    assert disagree > 0


@pytest.mark.parametrize("n", [1, 63, 65, 4095, 4097, 12289])
def test_expanded_tiles_and_ragged_tails(apd, orc, n):
    for d in (1, 2, 3, 8, 13, 33, 64):
        x = datagen.gaussian_blobs(n, d, seed=3000 * n + d, n_blobs=5,
                                   sigma=0.03, noise_frac=0.2)
        for offset in (0.0, 300.0):
            xo = (x + np.float32(offset)).astype(np.float32)
            eps = 0.05 * np.sqrt(d)
            want_l, want_c, _ = orc.fit(xo, eps, 4, form="expanded")
            for flags, mode in MODES[:2]:
                lab, cnt, _ = gpu_fit(apd, xo, eps, 4, flags=flags)
                assert_same(lab, cnt, want_l, want_c,
                            f"n={n} d={d} offset={offset} {mode}")


def test_expanded_edge_cases(apd, orc):
    """Far from the origin, ties at the radius, norms too large for the
    screen (every pair then takes the exact path, overflow included),
    subnormal scales, duplicates with eps = 0, an eps whose square
    overflows, 64-d data off the origin."""
    for name, x, eps in _screen_cases():
        for m in (1, 4):
            want_l, want_c, _ = orc.fit(x, eps, m, form="expanded")
            for flags in (EXP, EXP | 0x2):
                lab, cnt, _ = gpu_fit(apd, x, eps, m, flags=flags)
                assert_same(lab, cnt, want_l, want_c, f"{name} m={m} flags={flags}")


def test_expanded_rejects_pruning(apd):
    import torch
    x = torch.from_numpy(datagen.uniform_points(500, 3, 1)).cuda()
    with pytest.raises(apd.DbscanError) as e:
        apd.fit(x, 0.1, 3, flags=EXP | 0x4)
    assert e.value.status == -1
    with pytest.raises(apd.DbscanError) as e:
        apd.graph(x, 0.1, flags=EXP | 0x4)
    assert e.value.status == -1


def _golden():
    with open(os.path.join(pins.GOLDEN, "workloads.json")) as f:
        return json.load(f)


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a.astype("<i4")).tobytes()).hexdigest()


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_expanded_named_workload(apd, orc, key):
    x, eps, m, w = datagen.make_workload(key)
    print(f"workload {key} {w.name} expanded", flush=True)
    lab, cnt, info = gpu_fit(apd, x, eps, m, max_edges=1 << 30, flags=EXP)
    g = _golden().get(str(key), {})
    assert g.get("points_sha256") == datagen.sha256_points(x)
    ge = g.get("expanded")
    if ge is not None:
        assert _digest(cnt) == ge["counts_sha256"], "counts differ from the oracle"
        assert _digest(lab) == ge["labels_sha256"], "labels differ from the oracle"
        assert int(info["n_core"]) == ge["n_core"]
    rng = np.random.default_rng(500 + key)
    rows = rng.choice(w.n, size=min(w.n, 160), replace=False)
    assert np.array_equal(cnt[rows], orc.row_counts(x, eps, rows, form="expanded"))
    if key <= 2:
        want_l, want_c, _ = orc.fit(x, eps, m, form="expanded")
        assert_same(lab, cnt, want_l, want_c, w.name)


def test_expanded_graph(apd, orc):
    for x, eps, m in pins.far_cases(seed=141, count=12) + pins.small_cases(seed=143, count=20):
        want = orc.graph(x, eps, form="expanded")
        got_rp, got_ci, _ = gpu_graph(apd, x, eps, flags=EXP)
        assert_same_graph((got_rp, got_ci), want, f"n={x.shape} eps={eps}")
    for key in (1, 2, 3):
        x, eps, m, w = datagen.make_workload(key)
        rp, ci, _ = gpu_graph(apd, x, eps, flags=EXP)
        ge = _golden()[str(key)].get("expanded", {})
        if "graph_sha256" in ge:
            h = hashlib.sha256()
            h.update(np.ascontiguousarray(rp.astype("<i8")).tobytes())
            h.update(np.ascontiguousarray(ci.astype("<i4")).tobytes())
            assert h.hexdigest() == ge["graph_sha256"], w.name
        rng = np.random.default_rng(key)
        for i in rng.choice(w.n, size=8, replace=False):
            assert np.array_equal(ci[rp[i]:rp[i + 1]].astype(np.int64),
                                  orc.row_neighbours(x, eps, int(i), form="expanded"))
