"""The pruned count pass skips 64 rows against a wave's columns when their
boxes are provably farther apart than eps.  For wide points the gap sum is
formed by the whole wave (one dimension per lane, summed in a DPP tree)
and compared with a widened threshold (box_gap_threshold in
count_common.h): a tree sum above it must prove that the ascending-k fp32
sum of the same squared gaps, which bounds every pair's fp32 distance from
below, exceeds eps^2.

Checked here on the CPU with numpy float32 arithmetic in the kernel's own
orders, on gap vectors placed just above the threshold, and the threshold
without its widening is shown to fail the same check.
"""
import math

import numpy as np
import pytest

U = 2.0 ** -24


def box_gap_threshold(eps2, s, widen=True):
    """Host threshold of the wave box test (same formula as the library)."""
    if not widen:
        return np.float32(eps2)
    g = lambda m: m * U / (1.0 - m * U)
    t = float(eps2) * (1.0 + g(8.0)) / (1.0 - g(float(s))) * (1.0 + 2.0 ** -50)
    f = np.float32(t)
    if float(f) < t:
        f = np.nextafter(f, np.float32(np.inf))
    return f


def ordered_sum(q):
    s = q[0]
    for v in q[1:]:
        s = np.float32(s + v)
    return s


def tree_sum(q):
    """wave_sum_f32: 64 lanes (zeros past S), quad pairs, quads, halves and
    rows by DPP, then the four row sums left to right."""
    v = np.zeros(64, np.float32)
    v[:len(q)] = q
    for perm in ((lambda l: l ^ 1), (lambda l: l ^ 2),
                 (lambda l: (l & ~7) | (7 - (l & 7))),
                 (lambda l: (l & ~15) | (15 - (l & 15)))):
        v = np.array([np.float32(v[l] + v[perm(l)]) for l in range(64)], np.float32)
    r = [v[0], v[16], v[32], v[48]]
    return np.float32(np.float32(np.float32(r[0] + r[1]) + r[2]) + r[3])


def squared_gaps(g):
    return np.array([np.float32(x * x) for x in g.astype(np.float32)], np.float32)


def near_threshold_cases(s, eps2, rng, count):
    """Gap vectors whose tree sum lands just above the threshold: terms of
    mixed magnitude, rescaled so the sum sits at the bound, then nudged."""
    thr = float(box_gap_threshold(eps2, s))
    for _ in range(count):
        w = rng.random(s) ** rng.choice([1.0, 4.0, 16.0])
        g = np.sqrt(w / w.sum() * thr)
        g = g.astype(np.float32)
        for _ in range(64):
            q = squared_gaps(g)
            if tree_sum(q) > thr:
                yield q
                break
            k = rng.integers(s)
            g[k] = np.nextafter(g[k], np.float32(np.inf))


@pytest.mark.parametrize("s", [24, 32, 48, 64])
@pytest.mark.parametrize("eps", [0.35, 1e-3, 3.0e5])
def test_tree_sum_above_threshold_proves_the_ordered_sum(s, eps):
    eps2 = np.float32(np.float32(eps) * np.float32(eps))
    thr = box_gap_threshold(eps2, s)
    rng = np.random.default_rng(1000 * s + int(math.log10(eps) * 7 + 50))
    n = 0
    for q in near_threshold_cases(s, eps2, rng, 150):
        assert tree_sum(q) > thr
        assert ordered_sum(q) > eps2, (s, eps)
        n += 1
    assert n >= 100


def test_threshold_without_widening_is_caught():
    """With eps^2 itself as the threshold the tree sum can exceed it while
    the ordered sum does not: the widening is needed."""
    rng = np.random.default_rng(7)
    found = 0
    for s in (48, 64):
        eps2 = np.float32(np.float32(0.35) ** 2)
        for _ in range(3000):
            w = rng.random(s) ** 8
            g = np.sqrt(w / w.sum() * float(eps2)).astype(np.float32)
            q = squared_gaps(g)
            if tree_sum(q) > eps2 and not ordered_sum(q) > eps2:
                found += 1
                break
    assert found >= 1
