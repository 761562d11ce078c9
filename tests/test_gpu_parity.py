"""Parity of the HIP library (through the C ABI) with the brute-force oracle.

Labels and neighbour counts must be bit-identical.  Small and medium inputs
are compared element by element with a live oracle run; the five named
workloads at full size are compared with the oracle's stored SHA-256
digests (tests/golden/workloads.json, written by the oracle alone), with
sampled rows recomputed live by the oracle and with label invariants on
sampled points.
"""
import json
import os

import numpy as np
import pytest

import pins
from all_pairs_distance_amd import datagen

pytestmark = pytest.mark.gpu

GOLDEN_WORKLOADS = os.path.join(pins.GOLDEN, "workloads.json")


@pytest.fixture(scope="module")
def apd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import all_pairs_distance_amd
    return all_pairs_distance_amd


def gpu_fit(apd, x, eps, m, flags=0, max_edges=None):
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(-1, 1)
    n = x.shape[0]
    if max_edges is None:
        max_edges = max(1, min(n * (n - 1) // 2, 1 << 28))
    t = torch.from_numpy(x).cuda()
    labels, counts, info = apd.fit(t, eps, m, return_counts=True, flags=flags,
                                   max_edges=max_edges, return_info=True)
    torch.cuda.synchronize()
    return labels.cpu().numpy(), counts.cpu().numpy(), info


def assert_same(got_l, got_c, want_l, want_c, what):
    bad_c = np.nonzero(got_c != want_c)[0]
    assert bad_c.size == 0, f"{what}: {bad_c.size} counts differ, first {bad_c[:5]}"
    bad_l = np.nonzero(got_l != want_l)[0]
    assert bad_l.size == 0, f"{what}: {bad_l.size} labels differ, first {bad_l[:5]}"


# 2 = FLAG_FORCE_TILE_MERGE, 4 = FLAG_PRUNE_TILES, 8 = FLAG_SCREEN
MODES = [(0, "edges"), (2, "tiles"), (4, "pruned"), (6, "pruned_tiles"),
         (8, "screen"), (12, "pruned_screen"), (10, "screen_tiles")]


@pytest.mark.parametrize("flags,mode", MODES, ids=[m for _, m in MODES])
def test_handworked(apd, flags, mode):
    for cid, pts, eps, m, counts, labels in pins.load_handworked():
        lab, cnt, info = gpu_fit(apd, pts, eps, m, flags=flags)
        assert_same(lab, cnt, labels, counts, cid)


@pytest.mark.parametrize("flags,mode", MODES, ids=[m for _, m in MODES])
def test_small_random_vs_oracle(apd, orc, flags, mode):
    for t, (x, eps, m) in enumerate(pins.small_cases(seed=101, count=80)):
        want_l, want_c, _ = orc.fit(x, eps, m)
        lab, cnt, info = gpu_fit(apd, x, eps, m, flags=flags)
        assert_same(lab, cnt, want_l, want_c, f"case {t} n={x.shape} eps={eps} m={m}")
        if x.shape[0] > 0 and info["n_core"] > 0:
            want_mode = 2 if flags & 2 else 1
            assert info["merge_mode"] == want_mode


SIZES = [1, 2, 63, 64, 65, 255, 257, 4095, 4096, 4097, 8191, 12289]


@pytest.mark.parametrize("n", SIZES)
def test_tiles_and_ragged_tails(apd, orc, n):
    for d in (1, 2, 3, 5, 8, 13, 33, 64):
        x = datagen.gaussian_blobs(n, d, seed=1000 * n + d, n_blobs=5,
                                   sigma=0.03, noise_frac=0.2)
        eps = 0.05 * np.sqrt(d)
        want_l, want_c, _ = orc.fit(x, eps, 4)
        for flags, mode in MODES:
            lab, cnt, _ = gpu_fit(apd, x, eps, 4, flags=flags)
            assert_same(lab, cnt, want_l, want_c, f"n={n} d={d} {mode}")


def test_every_dimension(apd, orc):
    """Every d in 1..64: the compiled widths and the zero-padded ones."""
    for d in range(1, 65):
        x = datagen.gaussian_blobs(3000, d, seed=77 + d, n_blobs=6, sigma=0.02,
                                   noise_frac=0.1)
        eps = 0.04 * np.sqrt(d)
        want_l, want_c, _ = orc.fit(x, eps, 5)
        lab, cnt, _ = gpu_fit(apd, x, eps, 5)
        assert_same(lab, cnt, want_l, want_c, f"d={d}")
        lab, cnt, _ = gpu_fit(apd, x, eps, 5, flags=4)
        assert_same(lab, cnt, want_l, want_c, f"d={d} pruned")
        lab, cnt, _ = gpu_fit(apd, x, eps, 5, flags=8)
        assert_same(lab, cnt, want_l, want_c, f"d={d} screen")
        lab, cnt, _ = gpu_fit(apd, x, eps, 5, flags=12)
        assert_same(lab, cnt, want_l, want_c, f"d={d} pruned screen")


def test_multi_column_kernels_every_width(apd, orc):
    """Every width up to 16 at a size whose all-tiles pass runs the kernel
    with P = 16, 8, 4 or 2 column points per lane (512 or more work items;
    smaller sets take one point per lane), in the all-tiles, pruned and
    screened modes."""
    for d, n in ((1, 15000), (2, 15000), (3, 12000), (4, 12000), (6, 8000),
                 (8, 8000), (12, 6000), (16, 6000)):
        x = datagen.gaussian_blobs(n, d, seed=500 + d, n_blobs=5, sigma=0.03,
                                   noise_frac=0.1)
        eps = 0.02 * np.sqrt(d)
        want_l, want_c, _ = orc.fit(x, eps, 6)
        for flags in (0, 4, 8):
            lab, cnt, _ = gpu_fit(apd, x, eps, 6, flags=flags)
            assert_same(lab, cnt, want_l, want_c, f"d={d} n={n} flags={flags}")


def test_pruning_skips_tiles_exactly(apd, orc):
    """Well separated blobs: most block pairs are pruned, results equal."""
    for d, n in ((1, 60000), (2, 50000), (3, 40000), (8, 20000)):
        x = datagen.gaussian_blobs(n, d, seed=500 + d, n_blobs=40, sigma=0.004,
                                   noise_frac=0.05)
        eps = 0.01
        want_l, want_c, _ = orc.fit(x, eps, 6)
        lab, cnt, info = gpu_fit(apd, x, eps, 6, flags=4)
        assert_same(lab, cnt, want_l, want_c, f"d={d} n={n}")
        assert info["tiles_kept"] < info["tiles_total"]
        lab0, cnt0, info0 = gpu_fit(apd, x, eps, 6)
        assert info0["tiles_kept"] == info0["tiles_total"]
        assert info["n_edges"] == info0["n_edges"]
    # ties at the radius between blocks: integer lattice, eps exactly 1
    lat = datagen.integer_lattice(200, 2)
    want_l, want_c, _ = orc.fit(lat, 1.0, 5)
    lab, cnt, info = gpu_fit(apd, lat, 1.0, 5, flags=4)
    assert_same(lab, cnt, want_l, want_c, "lattice pruned")
    assert info["tiles_kept"] < info["tiles_total"]


def test_boundary_ties(apd, orc):
    """Distances that land exactly on eps^2, or one ulp either side."""
    x = datagen.collinear_chain(4000, 0.03)               # fl32(k * 0.03)
    for eps in (0.03, float(np.nextafter(np.float32(0.03), np.float32(1))),
                float(np.nextafter(np.float32(0.03), np.float32(0)))):
        want_l, want_c, _ = orc.fit(x, eps, 2)
        lab, cnt, _ = gpu_fit(apd, x, eps, 2)
        assert_same(lab, cnt, want_l, want_c, f"chain eps={eps!r}")
    lat = datagen.integer_lattice(40, 2)
    for eps, m in ((1.0, 5), (1.0, 4), (2.0 ** 0.5, 9), (0.0, 1)):
        want_l, want_c, _ = orc.fit(lat, eps, m)
        lab, cnt, _ = gpu_fit(apd, lat, eps, m)
        assert_same(lab, cnt, want_l, want_c, f"lattice eps={eps} m={m}")
    # subnormal squared differences are kept, not flushed
    x = np.array([[0.0], [1e-20], [3e-20]], np.float32)
    lab, cnt, _ = gpu_fit(apd, x, 0.0, 1)
    assert cnt.tolist() == [1, 1, 1] and lab.tolist() == [0, 1, 2]
    # ties and near-ties among subnormal squares with 16 column points per
    # lane (14,400 points: 640 work items), all tiles and pruned
    lat = (datagen.integer_lattice(120, 2) * np.float32(1e-20)).astype(np.float32)
    for eps in (1e-20, 1.5e-20):
        want_l, want_c, _ = orc.fit(lat, eps, 5)
        for flags in (0, 4):
            lab, cnt, _ = gpu_fit(apd, lat, eps, 5, flags=flags)
            assert_same(lab, cnt, want_l, want_c,
                        f"subnormal lattice eps={eps} flags={flags}")


def test_degenerate_inputs(apd, orc):
    same = np.ones((5000, 3), np.float32) * np.float32(0.25)
    lab, cnt, _ = gpu_fit(apd, same, 0.0, 5000)
    assert np.all(cnt == 5000) and np.all(lab == 0)
    lab, cnt, _ = gpu_fit(apd, same, 0.0, 5001)
    assert np.all(lab == -1)
    # a long chain: deep union-find paths, every point core
    chain = datagen.collinear_chain(100000, 0.5)
    lab, cnt, _ = gpu_fit(apd, chain, 0.5, 2)
    want_c = np.full(100000, 3, np.int32)
    want_c[[0, -1]] = 2
    assert np.array_equal(cnt, want_c) and np.all(lab == 0)
    lab, cnt, _ = gpu_fit(apd, chain, 0.5, 2, flags=2)
    assert np.array_equal(cnt, want_c) and np.all(lab == 0)
    # reversed chain: the smallest index sits at the far end
    rev = np.ascontiguousarray(chain[::-1])
    lab, _, _ = gpu_fit(apd, rev, 0.5, 3)
    assert lab[0] == 0 and lab[-1] == 0 and np.all(lab == 0)
    # MinPts = 1 and a radius larger than the diameter
    x = datagen.uniform_points(20000, 2, 5)
    lab, cnt, _ = gpu_fit(apd, x, 2.0, 1)
    assert np.all(cnt == 20000) and np.all(lab == 0)
    x = datagen.uniform_points(3000, 3, 6)
    want_l, want_c, _ = orc.fit(x, 0.05, 1)
    lab, cnt, _ = gpu_fit(apd, x, 0.05, 1)
    assert_same(lab, cnt, want_l, want_c, "minpts 1")


def test_concurrent_fits_on_two_streams(apd, orc):
    """Two host threads fit different sets at the same time, each on a
    stream and a workspace of its own (calls keep no state between them),
    three times each: every result equals its oracle."""
    import threading
    import torch
    x1, e1, m1, _ = datagen.make_workload(2)
    x2 = datagen.gaussian_blobs(30000, 3, seed=41, n_blobs=10, sigma=0.02,
                                noise_frac=0.1)
    sets = []
    for x, eps, m in ((x1, e1, m1), (x2, 0.02, 6)):
        want_l, want_c, _ = orc.fit(x, eps, m)
        sets.append((torch.from_numpy(x).cuda(), eps, m, want_l, want_c,
                     apd.Workspace(x.shape[0], x.shape[1], max_edges=1 << 26),
                     torch.cuda.Stream()))
    got = [[None] * 3 for _ in sets]
    errors = []

    def run(k):
        xt, eps, m, _, _, ws, st = sets[k]
        try:
            with torch.cuda.stream(st):
                for rep in range(3):
                    lab, cnt = apd.fit(xt, eps, m, return_counts=True,
                                       workspace=ws, stream=st)
                    got[k][rep] = (lab.cpu().numpy(), cnt.cpu().numpy())
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for k, (_, _, _, want_l, want_c, _, _) in enumerate(sets):
        for rep in range(3):
            lab, cnt = got[k][rep]
            assert_same(lab, cnt, want_l, want_c, f"set {k} call {rep}")


def test_narrow_radius_at_float_limits(apd, orc):
    """2-d points (16 column groups per lane) with squared distances that
    overflow to +inf.  eps = 1.8446744e19 squares to +inf (every pair is a
    neighbour, the pattern comes from ballots); eps = 1.8446743e19 squares
    to 3.4028233e38, the largest square of a float below +inf, so the
    float just above it is finite and overflowed pairs are not
    neighbours."""
    rng = np.random.default_rng(21)
    x = datagen.uniform_points(20000, 2, 22)   # 960 work items: P = 16
    far = rng.integers(0, 20000, 60)
    x[far, 0] = np.where(np.arange(60) % 2 == 0, np.float32(1.5e19),
                         np.float32(-1.5e19))
    for eps in (1.8446744e19, 1.8446743e19):
        with np.errstate(over="ignore"):
            e2 = np.float32(eps) * np.float32(eps)
        print(f"narrow eps {eps} eps2 {e2}", flush=True)
        want_l, want_c, _ = orc.fit(x, eps, 5)
        for flags in (0, 4):
            lab, cnt, _ = gpu_fit(apd, x, eps, 5, flags=flags)
            assert_same(lab, cnt, want_l, want_c, f"eps {eps} flags {flags}")
        if np.isinf(e2):
            assert np.all(want_c == 20000)
        else:
            assert want_c.min() < 20000


def test_pruned_key_sort_edge_cases(apd, orc):
    """The pruned mode's key sort on keys that are all equal, descending,
    or drawn from a few values: any permutation gives the same results,
    and a wrong one (a lost or repeated point) changes them."""
    prune = 4
    print("pruned sort: identical points", flush=True)
    same = np.ones((5000, 3), np.float32) * np.float32(0.25)
    lab, cnt, _ = gpu_fit(apd, same, 0.0, 5000, flags=prune)
    assert np.all(cnt == 5000) and np.all(lab == 0)
    print("pruned sort: ascending and descending chains", flush=True)
    chain = datagen.collinear_chain(100000, 0.5)
    want_c = np.full(100000, 3, np.int32)
    want_c[[0, -1]] = 2
    for pts in (chain, np.ascontiguousarray(chain[::-1])):
        lab, cnt, _ = gpu_fit(apd, pts, 0.5, 2, flags=prune)
        assert np.array_equal(cnt, want_c) and np.all(lab == 0)
    print("pruned sort: few distinct points, ragged sizes", flush=True)
    rng = np.random.default_rng(11)
    for n in (1023, 1025, 9000):
        sites = datagen.uniform_points(40, 2, 12)
        x = np.ascontiguousarray(sites[rng.integers(0, 40, n)])
        want_l, want_c, _ = orc.fit(x, 0.02, 30)
        lab, cnt, _ = gpu_fit(apd, x, 0.02, 30, flags=prune)
        assert_same(lab, cnt, want_l, want_c, f"few sites n={n}")


def test_edge_area_overflow_falls_back(apd, orc):
    x = datagen.gaussian_blobs(20000, 2, seed=3, n_blobs=4, sigma=0.05)
    want_l, want_c, _ = orc.fit(x, 0.02, 8)
    for cap in (0, 1, 1000):
        lab, cnt, info = gpu_fit(apd, x, 0.02, 8, max_edges=cap)
        assert info["merge_mode"] == 2
        assert_same(lab, cnt, want_l, want_c, f"cap={cap}")
    lab, cnt, info = gpu_fit(apd, x, 0.02, 8, max_edges=1 << 26)
    assert info["merge_mode"] == 1
    assert info["n_edges"] == (int(want_c.astype(np.int64).sum()) - 20000) // 2
    assert_same(lab, cnt, want_l, want_c, "edges")


def test_errors(apd):
    import torch
    x = datagen.uniform_points(1000, 3, 1)
    bad = x.copy()
    bad[500, 1] = np.nan
    with pytest.raises(apd.DbscanError) as e:
        gpu_fit(apd, bad, 0.1, 3)
    assert e.value.status == -2
    bad[500, 1] = np.inf
    with pytest.raises(apd.DbscanError) as e:
        gpu_fit(apd, bad, 0.1, 3)
    assert e.value.status == -2
    t = torch.from_numpy(x).cuda()
    lab = torch.empty(1000, dtype=torch.int32, device="cuda")
    need = apd.dbscan_workspace_bytes(1000, 3)
    ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    st = apd.dbscan_fit_device(t.data_ptr(), 1000, 3, 0.1, 3, lab.data_ptr(),
                               None, ws.data_ptr(), need - 256, None)
    assert st == -5
    st = apd.dbscan_fit_device(t.data_ptr(), 1000, 3, 0.1, 3, lab.data_ptr(),
                               None, ws.data_ptr() + 16, need, None)
    assert st == -5
    st = apd.dbscan_fit_device(t.data_ptr(), 1000, 3, 0.1, 3, lab.data_ptr(),
                               None, ws.data_ptr(), need, None)
    assert st == 0
    torch.cuda.synchronize()


def test_host_entry_and_optional_counts(apd, orc):
    import torch
    x = datagen.gaussian_blobs(9000, 4, seed=9, n_blobs=3, sigma=0.04)
    want_l, want_c, _ = orc.fit(x, 0.05, 6)
    lab, cnt = apd.fit_host(x, 0.05, 6, return_counts=True)
    assert_same(lab, cnt, want_l, want_c, "host entry")
    lab = apd.fit(torch.from_numpy(x).cuda(), 0.05, 6).cpu().numpy()
    assert np.array_equal(lab, want_l)
    # n = 0 is a no-op
    assert apd.fit_host(np.zeros((0, 3), np.float32), 0.1, 1).size == 0


def test_repeatable(apd):
    x, eps, m, _ = datagen.make_workload(2)
    first = gpu_fit(apd, x, eps, m)
    for _ in range(5):
        again = gpu_fit(apd, x, eps, m)
        assert np.array_equal(first[0], again[0])
        assert np.array_equal(first[1], again[1])


def _golden():
    if not os.path.exists(GOLDEN_WORKLOADS):
        return {}
    with open(GOLDEN_WORKLOADS) as f:
        return json.load(f)


def _digest(a):
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(a.astype("<i4")).tobytes()).hexdigest()


NAMED_MODES = [(0, "all_tiles"), (4, "pruned"), (8, "screen"),
               (12, "pruned_screen")]


@pytest.mark.parametrize("flags,mode", NAMED_MODES,
                         ids=[m for _, m in NAMED_MODES])
@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_named_workload(apd, orc, key, flags, mode):
    x, eps, m, w = datagen.make_workload(key)
    print(f"workload {key} {w.name} {mode}", flush=True)
    lab, cnt, info = gpu_fit(apd, x, eps, m, max_edges=1 << 30, flags=flags)
    assert info["merge_mode"] == 1
    # full-size parity: every count and every label against the oracle's
    # stored digests, for exactly these input bytes (no fallback)
    g = _golden().get(str(key))
    assert g is not None, f"no oracle digests stored for workload {key}"
    assert g["points_sha256"] == datagen.sha256_points(x), \
        "the generator's output changed since the oracle digests were written"
    assert _digest(cnt) == g["counts_sha256"], "counts differ from the oracle"
    assert _digest(lab) == g["labels_sha256"], "labels differ from the oracle"
    assert int(info["n_core"]) == g["n_core"]
    # rows recomputed by the oracle right now
    rng = np.random.default_rng(key)
    rows = rng.choice(w.n, size=min(w.n, 192), replace=False)
    want = orc.row_counts(x, eps, rows)
    assert np.array_equal(cnt[rows], want)
    # invariants on sampled points, with core flags from the oracle: a core
    # point shares its label with (a sample of) its core neighbours; a
    # border point carries the label of its lowest-index core neighbour;
    # noise has no core neighbour
    for i in rng.choice(w.n, size=6, replace=False):
        nb = orc.row_neighbours(x, eps, int(i))
        assert nb.size == cnt[i]
        if cnt[i] >= m:
            some = rng.choice(nb, size=min(nb.size, 32), replace=False)
            some_core = some[orc.row_counts(x, eps, some) >= m]
            assert np.all(lab[some_core] == lab[i])
        else:
            lowest = None
            for k in range(0, nb.size, 16):
                part = nb[k:k + 16]
                hit = part[orc.row_counts(x, eps, part) >= m]
                if hit.size:
                    lowest = int(hit.min())
                    break
            assert lab[i] == (-1 if lowest is None else lab[lowest])
        if lab[i] != -1:
            assert lab[i] <= i and lab[lab[i]] == lab[i]
    if key <= 2:   # small enough for a live full oracle run
        want_l, want_c, _ = orc.fit(x, eps, m)
        assert_same(lab, cnt, want_l, want_c, w.name)


@pytest.mark.parametrize("key", [1, 2, 3])
def test_named_workload_tile_merge(apd, key):
    x, eps, m, w = datagen.make_workload(key)
    a = gpu_fit(apd, x, eps, m, max_edges=1 << 30)
    b = gpu_fit(apd, x, eps, m, flags=2)
    assert b[2]["merge_mode"] == 2 and b[2]["pass2_pairs"] > 0
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _screen_cases():
    """Inputs that push the screened count pass onto its exact path: data
    far from the origin (a wide bound), ties exactly at the radius away
    from the origin, norms too large for the bound, subnormal scales,
    duplicates with eps = 0, and an eps whose square overflows."""
    rng = np.random.default_rng(77)
    out = []
    blobs = datagen.gaussian_blobs(3000, 3, seed=71, n_blobs=6, sigma=0.02,
                                   noise_frac=0.1)
    out.append(("far_from_origin", (blobs + np.float32(1000.0)).astype(np.float32), 0.03))
    out.append(("offset_1e6", (blobs + np.float32(1e6)).astype(np.float32), 0.5))
    lat = datagen.integer_lattice(40, 3).astype(np.float32)
    out.append(("lattice_ties_offset", (lat + np.float32(37.0)).astype(np.float32), 1.0))
    out.append(("lattice_ties_diag", (lat * np.float32(0.25) - np.float32(3.0)).astype(np.float32),
                float(np.sqrt(np.float32(0.125)))))
    huge = datagen.uniform_points(2000, 4, 5) * np.float32(2.0 ** 60)
    out.append(("huge_norms", huge.astype(np.float32), float(2.0 ** 57)))
    tiny = datagen.uniform_points(2000, 2, 6) * np.float32(1e-38)
    out.append(("subnormal_scale", tiny.astype(np.float32), 2e-40))
    base = datagen.uniform_points(300, 8, 7)
    dup = np.ascontiguousarray(base[rng.integers(0, 300, 2500)])
    out.append(("duplicates_eps0", dup, 0.0))
    out.append(("eps_square_overflows", datagen.uniform_points(1500, 2, 8), 3e19))
    wide = datagen.gaussian_blobs(2500, 64, seed=72, n_blobs=5, sigma=0.05,
                                  noise_frac=0.1)
    out.append(("d64_offset", (wide + np.float32(20.0)).astype(np.float32), 0.4))
    return out


@pytest.mark.parametrize("flags,mode", [(8, "screen"), (12, "pruned_screen")],
                         ids=["screen", "pruned_screen"])
def test_screen_edge_cases(apd, orc, flags, mode):
    for name, x, eps in _screen_cases():
        for m in (1, 4):
            want_l, want_c, _ = orc.fit(x, eps, m)
            lab, cnt, _ = gpu_fit(apd, x, eps, m, flags=flags)
            assert_same(lab, cnt, want_l, want_c, f"{name} m={m}")


def test_schedule_shake(apd, orc):
    """Walking the count pass's items, the recorded pairs and the tile
    merge's blocks in reverse order or in seeded shuffled orders (and with
    another edge capacity, which changes which merge runs and the order
    pairs are recorded in) gives the same labels: the union-find result
    does not depend on the order of the links."""
    cases = [(datagen.collinear_chain(20000, 0.5), 0.5, 2),
             (datagen.integer_lattice(120, 2), 1.0, 5),
             (datagen.gaussian_blobs(30000, 3, seed=9, n_blobs=30, sigma=0.01,
                                     noise_frac=0.1), 0.012, 6)]
    x2, e2, m2, _ = datagen.make_workload(2)
    cases.append((x2, e2, m2))
    # wide points: the screened pass runs on the matrix cores
    cases.append((datagen.gaussian_blobs(9000, 48, seed=19, n_blobs=8,
                                         sigma=0.05, noise_frac=0.1), 0.45, 5))
    for x, eps, m in cases:
        want_l, want_c, _ = orc.fit(x, eps, m)
        shuffles = tuple(0x40 | (seed << 16) for seed in (0, 1, 7, 123, 4321, 65535))
        for base in (0, 2, 4, 8, 12):
            for fl in (base, base | 0x10) + tuple(base | sh for sh in shuffles):
                lab, cnt, _ = gpu_fit(apd, x, eps, m, flags=fl)
                assert_same(lab, cnt, want_l, want_c, f"n={x.shape} flags={fl}")
        lab, cnt, info = gpu_fit(apd, x, eps, m, flags=0x10, max_edges=1000)
        assert info["merge_mode"] == 2
        assert_same(lab, cnt, want_l, want_c, f"n={x.shape} small edge area")


def test_relabel_contiguous(apd, orc):
    import torch
    for t, (x, eps, m) in enumerate(pins.small_cases(seed=303, count=30)):
        lab, _, _ = orc.fit(x, eps, m)
        want_ids, want_sizes, k = orc.relabel(lab)
        ids, sizes = apd.relabel(torch.from_numpy(lab).cuda())
        assert np.array_equal(ids.cpu().numpy(), want_ids), t
        assert np.array_equal(sizes.cpu().numpy(), want_sizes), t
    for key in (2, 3):
        x, eps, m, w = datagen.make_workload(key)
        lab, _, _ = gpu_fit(apd, x, eps, m, max_edges=1 << 28)
        want_ids, want_sizes, k = orc.relabel(lab)
        ids, sizes = apd.relabel(torch.from_numpy(lab).cuda())
        assert np.array_equal(ids.cpu().numpy(), want_ids), w.name
        assert np.array_equal(sizes.cpu().numpy(), want_sizes), w.name
    bad = torch.tensor([0, 0, 5, -1], dtype=torch.int32, device="cuda")
    with pytest.raises(apd.DbscanError) as e:
        apd.relabel(bad)
    assert e.value.status == -1


def test_random_sets_every_mode_and_walk(apd, orc):
    """Seeded random blob sets across the compiled widths, sizes on both
    sides of the small-set switch and of the pruning box tests, in every
    count mode and under shuffled work orders: labels and counts must equal
    the oracle's (the hoisted-norm mode: the oracle's hoisted-norm form)."""
    rng = np.random.default_rng(2026)
    for case in range(24):
        d = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64]))
        n = int(rng.choice([50, 700, 2000, 4097, 9000, 15000]))
        x = datagen.gaussian_blobs(n, d, seed=int(rng.integers(1 << 30)),
                                   n_blobs=int(rng.integers(2, 8)),
                                   sigma=float(rng.uniform(0.01, 0.06)),
                                   noise_frac=float(rng.uniform(0, 0.3)))
        eps = float(rng.uniform(0.02, 0.12)) * float(np.sqrt(d))
        m = int(rng.integers(1, 12))
        want_l, want_c, _ = orc.fit(x, eps, m)
        for fl, mode in ((0, "all_tiles"), (4, "pruned"), (8, "screen"),
                         (12, "pruned_screen")):
            for seed in (0, 5):
                flags = fl | ((0x40 | (seed << 16)) if seed else 0)
                lab, cnt, _ = gpu_fit(apd, x, eps, m, flags=flags)
                assert_same(lab, cnt, want_l, want_c,
                            f"case {case} n={n} d={d} {mode} seed={seed}")
        want_l, want_c, _ = orc.fit(x, eps, m, form="expanded")
        lab, cnt, _ = gpu_fit(apd, x, eps, m, flags=0x20)
        assert_same(lab, cnt, want_l, want_c, f"case {case} n={n} d={d} expanded")
