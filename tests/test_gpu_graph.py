"""Parity of the sparse eps-graph export (dbscan_graph_device, through the C
ABI) with the oracle's CSR graph.

Row offsets and column indices must be bit-identical: every row lists the
point itself and all neighbours within eps in ascending order, so the
result is unique.  Small inputs are compared with a live oracle run; the
named workloads at full size with the oracle's stored digest, with sampled
rows recomputed live by the oracle, and with structure checks.
"""
import ctypes
import hashlib
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


def gpu_graph(apd, x, eps, flags=0, max_pairs=None):
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(-1, 1)
    t = torch.from_numpy(x).cuda()
    row_ptr, col_idx, info = apd.graph(t, eps, flags=flags, max_pairs=max_pairs,
                                       return_info=True)
    torch.cuda.synchronize()
    return row_ptr.cpu().numpy(), col_idx.cpu().numpy(), info


def assert_same_graph(got, want, what):
    rp, ci = got
    wrp, wci = want
    assert rp.shape == wrp.shape, what
    bad = np.nonzero(rp != wrp)[0]
    assert bad.size == 0, f"{what}: {bad.size} row offsets differ, first {bad[:5]}"
    assert ci.shape == wci.shape, what
    bad = np.nonzero(ci != wci)[0]
    assert bad.size == 0, f"{what}: {bad.size} column entries differ, first {bad[:5]}"


MODES = [(0, "all_tiles"), (4, "pruned"), (8, "screen"), (12, "pruned_screen")]


def test_graph_handworked(apd):
    for cid, x, eps, rp, ci in pins.load_graph_cases():
        for flags, mode in MODES:
            got_rp, got_ci, _ = gpu_graph(apd, x, eps, flags=flags)
            assert_same_graph((got_rp, got_ci), (rp, ci), f"{cid} {mode}")


@pytest.mark.parametrize("flags,mode", MODES, ids=[m for _, m in MODES])
def test_graph_small_random_vs_oracle(apd, orc, flags, mode):
    for t, (x, eps, m) in enumerate(pins.small_cases(seed=131, count=60)):
        want = orc.graph(x, eps)
        got_rp, got_ci, info = gpu_graph(apd, x, eps, flags=flags)
        assert_same_graph((got_rp, got_ci), want, f"case {t} n={x.shape} eps={eps}")


def test_graph_long_and_mixed_rows(apd, orc):
    """Rows of every length class of the row sort: a shuffled integer line
    (point p at position perm[p]) with eps = 4500 gives rows of 4,501 to
    9,001 entries (the merge passes after the 4,096-entry chunks: one pass
    near the ends of the line, two in the middle), and a second, sparse
    line gives rows of 1 to 3 entries (one wave per row); blobs in between
    give rows of a few dozen to a few hundred entries."""
    rng = np.random.default_rng(4242)
    dense = rng.permutation(9000).astype(np.float32)
    sparse = (1.0e6 + 4000.0 * rng.permutation(3000)).astype(np.float32)
    mid = (1.4e7 + rng.uniform(0.0, 2.0e5, 4000)).astype(np.float32)
    x = np.concatenate([dense, sparse, mid])
    x = np.ascontiguousarray(x[rng.permutation(x.size)]).reshape(-1, 1)
    want = orc.graph(x, 4500.0)
    lengths = np.diff(want[0])
    assert lengths.max() > 8192 and lengths.min() <= 3
    assert np.any((lengths > 2) & (lengths <= 64))
    assert np.any((lengths > 4096) & (lengths <= 8192))
    assert np.any((lengths > 64) & (lengths <= 4096))
    for flags, mode in ((0, "all_tiles"), (4, "pruned")):
        got_rp, got_ci, _ = gpu_graph(apd, x, 4500.0, flags=flags)
        assert_same_graph((got_rp, got_ci), want, f"long rows {mode}")


@pytest.mark.parametrize("n", [491520, 491521, 509500])
def test_graph_long_rows_at_the_bitmap_limit(apd, orc, n):
    """Long rows on both sides of the LDS bitmap sort's limit: up to 491,520
    points (a 60 KB bitmap) the bitmap, above it the work-group networks
    and merges.  9,000 points on an integer line (eps = 4,500: rows of
    4,501 to 9,001 entries) and the rest isolated points on a grid of pitch
    5,000, well away from it.
    Integer coordinates below 2^22 make every fp32 decision exact (a pair
    of the line is a neighbour iff its positions differ by at most 4,500,
    a grid point only neighbours itself), so every row is checked against
    that closed form, as the oracle's own one-dimensional pin does; sampled
    rows are also recomputed by the oracle (its all-pairs graph at this
    size would take minutes)."""
    rng = np.random.default_rng(777)
    nd = 9000
    line = np.stack([rng.permutation(nd).astype(np.float64), np.zeros(nd)], 1)
    gx, gy = np.meshgrid(np.arange(715), np.arange(700))
    grid = np.stack([20000.0 + 5000.0 * gx.ravel(), 5000.0 + 5000.0 * gy.ravel()], 1)
    x = np.concatenate([line, grid[:n - nd]]).astype(np.float32)
    x = np.ascontiguousarray(x[rng.permutation(len(x))])
    eps = 4500.0
    assert len(x) == n
    on_line = x[:, 1] == 0.0
    line_idx = np.nonzero(on_line)[0]
    by_pos = np.empty(nd, np.int64)
    by_pos[x[line_idx, 0].astype(np.int64)] = line_idx
    lo = np.maximum(np.arange(nd) - 4500, 0)
    hi = np.minimum(np.arange(nd) + 4500, nd - 1)
    want_len = np.ones(n, np.int64)
    want_len[by_pos] = hi - lo + 1
    assert want_len.max() > 8192
    for flags, mode in ((0, "all_tiles"), (4, "pruned")):
        rp, ci, _ = gpu_graph(apd, x, eps, flags=flags)
        assert rp[0] == 0 and np.array_equal(np.diff(rp), want_len), mode
        single = np.nonzero(~on_line)[0]
        assert np.array_equal(ci[rp[single]], single), mode
        for p in range(nd):
            i = by_pos[p]
            want = np.sort(by_pos[lo[p]:hi[p] + 1])
            assert np.array_equal(ci[rp[i]:rp[i + 1]], want), (mode, p)
        for i in (by_pos[0], by_pos[4500], by_pos[8999], single[0], single[-1]):
            got = ci[rp[i]:rp[i + 1]].astype(np.int64)
            assert np.array_equal(got, orc.row_neighbours(x, eps, int(i))), (mode, i)


@pytest.mark.parametrize("n", [1, 63, 65, 4095, 4097, 12289])
def test_graph_tiles_and_ragged_tails(apd, orc, n):
    for d in (1, 2, 3, 8, 33, 64):
        x = datagen.gaussian_blobs(n, d, seed=2000 * n + d, n_blobs=5,
                                   sigma=0.03, noise_frac=0.2)
        eps = 0.05 * np.sqrt(d)
        want = orc.graph(x, eps)
        for flags, mode in MODES:
            got_rp, got_ci, _ = gpu_graph(apd, x, eps, flags=flags)
            assert_same_graph((got_rp, got_ci), want, f"n={n} d={d} {mode}")


def test_graph_degenerate(apd, orc):
    import torch
    # no points: row_ptr = [0]
    rp, ci, _ = gpu_graph(apd, np.zeros((0, 3), np.float32), 0.1)
    assert rp.tolist() == [0] and ci.size == 0
    # one point
    rp, ci, _ = gpu_graph(apd, np.ones((1, 5), np.float32), 0.0)
    assert rp.tolist() == [0, 1] and ci.tolist() == [0]
    # every point a duplicate of every other: the complete graph
    x = np.full((3000, 2), 0.25, np.float32)
    rp, ci, _ = gpu_graph(apd, x, 0.0)
    assert np.array_equal(rp, np.arange(3001, dtype=np.int64) * 3000)
    assert np.array_equal(ci, np.tile(np.arange(3000, dtype=np.int32), 3000))
    # eps = 0 with some duplicates, and eps wide enough for one component
    rng = np.random.default_rng(5)
    base = datagen.uniform_points(700, 3, 9)
    x = np.ascontiguousarray(base[rng.integers(0, 700, 2000)])
    for eps in (0.0, 2.0):
        assert_same_graph(gpu_graph(apd, x, eps)[:2], orc.graph(x, eps),
                          f"duplicates eps={eps}")
    # a non-finite coordinate is an error
    bad = datagen.uniform_points(100, 2, 3)
    bad[17, 1] = np.inf
    with pytest.raises(apd.DbscanError) as e:
        apd.graph(torch.from_numpy(bad).cuda(), 0.1)
    assert e.value.status == -2


def test_graph_sizes_reported(apd, orc):
    """A call whose buffers are too small reports the sizes and leaves the
    row offsets valid; a second call with those sizes succeeds."""
    import torch
    c = apd._c()
    x = datagen.gaussian_blobs(5000, 3, seed=61, n_blobs=4, sigma=0.02,
                               noise_frac=0.1)
    eps = 0.03
    want_rp, want_ci = orc.graph(x, eps)
    nnz_want = int(want_rp[-1])
    pairs_want = (nnz_want - 5000) // 2
    t = torch.from_numpy(x).cuda()
    stream = torch.cuda.current_stream().cuda_stream
    row_ptr = torch.empty(5001, dtype=torch.int64, device="cuda")

    def call(col_cap, max_pairs, with_col=True):
        ws = torch.empty(c.dbscan_graph_workspace_bytes(5000, 3, max_pairs),
                         dtype=torch.uint8, device="cuda")
        col = torch.empty(max(col_cap, 1), dtype=torch.int32, device="cuda")
        nnz = ctypes.c_int64(-1)
        info = c.dbscan_info()
        st = c.dbscan_graph_device(
            t.data_ptr(), 5000, 3, eps, row_ptr.data_ptr(),
            col.data_ptr() if with_col else None, col_cap, nnz, ws.data_ptr(),
            ws.numel(), stream, 0, info)
        torch.cuda.synchronize()
        return st, nnz.value, info, col

    # size query: no column buffer at all
    st, nnz, info, _ = call(0, 0, with_col=False)
    assert st == c.ERR_CAPACITY and nnz == nnz_want
    assert info.n_edges == pairs_want
    assert np.array_equal(row_ptr.cpu().numpy(), want_rp)
    # column buffer one entry short
    st, nnz, info, _ = call(nnz_want - 1, pairs_want)
    assert st == c.ERR_CAPACITY and nnz == nnz_want
    # columns fit, pairs do not fit the workspace (its size is rounded up,
    # so ask for clearly fewer pairs than needed)
    st, nnz, info, _ = call(nnz_want, pairs_want // 2)
    assert st == c.ERR_WORKSPACE and nnz == nnz_want
    assert info.n_edges == pairs_want and info.edge_capacity < pairs_want
    assert np.array_equal(row_ptr.cpu().numpy(), want_rp)
    # exact sizes
    st, nnz, info, col = call(nnz_want, pairs_want)
    assert st == 0 and nnz == nnz_want
    assert np.array_equal(row_ptr.cpu().numpy(), want_rp)
    assert np.array_equal(col[:nnz].cpu().numpy(), want_ci)
    # the Python wrapper retries once with the reported sizes
    rp, ci, info = gpu_graph(apd, x, eps, max_pairs=10)
    assert_same_graph((rp, ci), (want_rp, want_ci), "retry")


def _golden():
    with open(GOLDEN_WORKLOADS) as f:
        return json.load(f)


def _graph_digest(row_ptr, col_idx):
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(row_ptr.astype("<i8")).tobytes())
    h.update(np.ascontiguousarray(col_idx.astype("<i4")).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("flags,mode", MODES, ids=[m for _, m in MODES])
@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_graph_named_workload(apd, orc, key, flags, mode):
    x, eps, m, w = datagen.make_workload(key)
    print(f"workload {key} {w.name} {mode}", flush=True)
    rp, ci, info = gpu_graph(apd, x, eps, flags=flags)
    g = _golden().get(str(key))
    assert g is not None and g["points_sha256"] == datagen.sha256_points(x)
    # row lengths are the oracle's neighbour counts
    counts = np.diff(rp).astype("<i4")
    assert hashlib.sha256(counts.tobytes()).hexdigest() == g["counts_sha256"]
    assert int(rp[-1]) == g["sum_counts"]
    if "graph_sha256" in g:
        assert _graph_digest(rp, ci) == g["graph_sha256"], "graph differs from the oracle"
    # rows recomputed by the oracle right now, and symmetry on those rows
    rng = np.random.default_rng(100 + key)
    for i in rng.choice(w.n, size=12, replace=False):
        row = ci[rp[i]:rp[i + 1]]
        assert np.array_equal(row.astype(np.int64), orc.row_neighbours(x, eps, int(i)))
        for j in row[:: max(1, row.size // 16)]:
            other = ci[rp[j]:rp[j + 1]]
            k = np.searchsorted(other, i)
            assert k < other.size and other[k] == i
    if key <= 2:   # small enough for a live full oracle run
        assert_same_graph((rp, ci), orc.graph(x, eps), w.name)
