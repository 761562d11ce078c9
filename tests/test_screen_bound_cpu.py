"""The screened count pass decides a pair without the exact distance only
when its rounding-error bound proves the exact fp32 decision.  This checks
that claim on the CPU, with exact rational arithmetic, on pairs placed
just inside and just outside the radius, far from and near the origin.

The screen value and the two per-point thresholds are recomputed here the
way the screen-table and count kernels define them (the fused multiply-add
chain is evaluated exactly and rounded once per step); the exact decision
is the direct fp32 distance of the rational model in pins.py.  Every pair
the screen settles must agree with it.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import pins

WIDTHS = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64)


def compiled_width(d):
    return next(w for w in WIDTHS if w >= d)


def fma32(a, b, c):
    return np.float32(float(pins.rn32(Fraction(float(a)) * Fraction(float(b))
                                      + Fraction(float(c)))))


def sq_norm64(p):
    s = 0.0
    for v in np.asarray(p, np.float32):
        s += float(v) * float(v)        # fp64, ascending, like the kernel
    return s


def round_down32(v):
    f = np.float32(v)
    if np.isfinite(f) and float(f) > v:
        f = np.nextafter(f, np.float32(-np.inf))
    return f


def round_up32(v):
    f = np.float32(v)
    if np.isfinite(f) and float(f) < v:
        f = np.nextafter(f, np.float32(np.inf))
    return f


def thresholds(x2, Y, eps2, D, kap_scale=1.0):
    u, t = 2.0 ** -24, 2.0 ** -149
    gD = D * u / (1 - D * u)
    g2 = (D + 2) * u / (1 - (D + 2) * u)
    kap = (u + 2.01 * gD) * kap_scale
    e2 = float(eps2)
    L = (e2 - (D + 2) * t) / (1 + g2)
    H = (e2 + (D + 2) * t) / (1 - g2)
    m = kap * (x2 + Y) + (D + 1) * t + 1e-12 * (abs(L) + abs(H) + x2 + Y)
    return round_down32(L - x2 - m), round_up32(H - x2 + m)


def screen_value(x, y):
    v = np.float32(sq_norm64(y))        # n_y, rounded to nearest
    for xk, yk in zip(x, y):
        v = fma32(np.float32(-2.0) * xk, yk, v)
    return v


def near_radius_pairs(rng, d, scale, eps, count):
    """Pairs whose real distance is eps times (1 +- beta), beta from 1e-7
    to 0.5 (log-uniform), centred at random points of norm up to `scale`;
    plus an exact duplicate."""
    out = []
    for _ in range(count):
        x = (rng.uniform(-1, 1, d) * scale).astype(np.float32)
        u = rng.normal(size=d)
        u /= np.linalg.norm(u)
        beta = 10.0 ** rng.uniform(-7, -0.3) * rng.choice([-1.0, 1.0])
        y = (x.astype(np.float64) + eps * (1 + beta) * u).astype(np.float32)
        out.append((x, y))
    out.append((out[0][0], out[0][0].copy()))
    return out


def check_pairs(pairs, eps, D, kap_scale=1.0):
    eps2 = pins.eps2_of(eps)
    # the set's largest squared norm, as the first screen kernel finds it
    Y = max(max(sq_norm64(x), sq_norm64(y)) for x, y in pairs)
    settled = {"in": 0, "out": 0, "exact": 0, "wrong": 0}
    for x, y in pairs:
        lo, hi = thresholds(sq_norm64(x), Y, eps2, D, kap_scale)
        v = screen_value(x, y)
        exact = pins.exact_d2_rounded(x, y) <= eps2
        if v <= lo:
            settled["in"] += 1
            settled["wrong"] += not exact
        elif v > hi:
            settled["out"] += 1
            settled["wrong"] += bool(exact)
        else:
            settled["exact"] += 1
    return settled


CASES = [(1, 1.0, 0.01), (2, 1.0, 0.003), (3, 1.0, 0.003), (3, 100.0, 0.05),
         (3, 1e4, 2.0), (8, 1.0, 0.05), (16, 3.0, 0.2), (64, 1.0, 0.35),
         (64, 30.0, 1.0)]


@pytest.mark.parametrize("d,scale,eps", CASES)
def test_screen_decisions_agree_with_the_exact_distance(d, scale, eps):
    rng = np.random.default_rng(1000 * d + int(scale))
    pairs = near_radius_pairs(rng, d, scale, eps, 300 if d < 32 else 100)
    settled = check_pairs(pairs, eps, compiled_width(d))
    assert settled["wrong"] == 0, settled
    # pairs far enough from the radius are settled by the screen itself
    if scale <= 3.0:
        assert settled["in"] > 1 and settled["out"] > 0, settled
    assert settled["exact"] > 0, settled


def test_a_bound_without_the_rounding_terms_is_caught():
    """The same pairs expose thresholds that ignore the screen's rounding
    error (kappa = 0): some pair is then settled the wrong way."""
    wrong = 0
    for d, scale, eps in CASES:
        rng = np.random.default_rng(1000 * d + int(scale))
        pairs = near_radius_pairs(rng, d, scale, eps, 300 if d < 32 else 100)
        wrong += check_pairs(pairs, eps, compiled_width(d), kap_scale=0.0)["wrong"]
    assert wrong > 0


def test_threshold_rounding_is_outward():
    for v in (1e-3, -2.5, 3.0000001, 1e-40, -1e-40, 1e39, -1e39):
        lo, hi = round_down32(v), round_up32(v)
        assert float(lo) <= v <= float(hi) or (math.isinf(float(hi)) and v > 0) \
            or (math.isinf(float(lo)) and v < 0)
