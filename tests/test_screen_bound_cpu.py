"""The screened count pass decides a pair without the exact distance only
when its rounding-error bound proves the exact fp32 decision.  This checks
that claim on the CPU, with exact rational arithmetic, on pairs placed
just inside and just outside the radius, far from and near the origin.

The screen value and the two per-point thresholds are recomputed here the
way the screen-table and count kernels define them (the fused multiply-add
chain is evaluated exactly and rounded once per step); the exact decision
is the direct fp32 distance of the rational model in pins.py.  Every pair
the screen settles must agree with it.

For the screen on the matrix cores (widths 16 and up), whose summation
order, product rounding and rounding mode are not specified, the products'
sum is formed under several such models, each exactly, the norm added
last by one rounded fp32 addition, against the thresholds of that path.  With the hoisted-norm form as the
decision, the thresholds of that mode are checked against that form's
exact value (pins.exact_expanded_rounded) the same way.
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


def thresholds(x2, Y, eps2, D, kap_scale=1.0, matrix=False, expanded=False,
               form_scale=1.0):
    """lo and hi of one row as the screen-table kernel computes them; with
    `expanded` for the hoisted-norm form as the decision (its own error
    term scaled by form_scale)."""
    u, t = 2.0 ** -24, 2.0 ** -149
    gD = D * u / (1 - D * u)
    g2 = (D + 2) * u / (1 - (D + 2) * u)
    gM = 2 * D * u / (1 - 2 * D * u)
    kap = ((1.01 * gM + 3.01 * u * (1 + gM)) if matrix else (u + 2.01 * gD)) * kap_scale
    flush = (2 * D + 2) * 2.0 ** -126 * (1 + 2 * math.sqrt(Y)) * kap_scale if matrix else 0.0
    e2 = float(eps2)
    if expanded:
        kapE = (u + 2.01 * gD) * form_scale
        m = (kap + kapE) * (x2 + Y) + 4 * (D + 1) * t + flush + 1e-12 * (e2 + x2 + Y)
        return (round_down32(e2 - x2 - m),
                round_up32(e2 * (1 + 2 * u) + 2 * t - x2 + m))
    L = (e2 - (D + 2) * t) / (1 + g2)
    H = (e2 + (D + 2) * t) / (1 - g2)
    m = kap * (x2 + Y) + (D + 1) * t + flush + 1e-12 * (abs(L) + abs(H) + x2 + Y)
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


def round32(q, mode):
    """A rational rounded to binary32 (gradual underflow) to nearest ("rn"),
    toward zero ("rz"), up ("ru") or down ("rd")."""
    r = pins.rn32(q)
    if mode == "rn" or r == q:
        return r
    if mode == "rz":
        mode = "rd" if q > 0 else "ru"
    f = np.float32(float(r))
    if mode == "ru" and r < q:
        return Fraction(float(np.nextafter(f, np.float32(np.inf))))
    if mode == "rd" and r > q:
        return Fraction(float(np.nextafter(f, np.float32(-np.inf))))
    return r


def matrix_screen_value(x, y, D, mode, fused, order):
    """The screen value as the count pass forms it on a matrix unit: D/4
    instructions accumulate from zero, instruction t adding the products
    of dims q*D/4 + t, q = 0..3 (one per lane group), as a matrix unit
    might: products exact or rounded on their own; the four additions of
    an instruction in order, reversed, as a tree, or with one rounding;
    every rounding in `mode`.  Then n_y is added by one fp32 addition
    rounded to nearest."""
    kq = D // 4
    a = [Fraction(float(np.float32(-2.0) * v)) for v in x] + [Fraction(0)] * (D - len(x))
    b = [Fraction(float(v)) for v in y] + [Fraction(0)] * (D - len(y))
    prods = [ak * bk for ak, bk in zip(a, b)]
    if not fused:
        prods = [round32(p, mode) for p in prods]
    acc = Fraction(0)
    for t in range(kq):
        grp = [prods[qq * kq + t] for qq in range(4)]
        if order == "seq":
            for p in grp:
                acc = round32(acc + p, mode)
        elif order == "rev":
            for p in reversed(grp):
                acc = round32(acc + p, mode)
        elif order == "tree":
            s01 = round32(grp[0] + grp[1], mode)
            s23 = round32(grp[2] + grp[3], mode)
            acc = round32(acc + round32(s01 + s23, mode), mode)
        else:   # "wide": the instruction's sum rounded once
            acc = round32(acc + sum(grp), mode)
    return round32(acc + Fraction(float(np.float32(sq_norm64(y)))), "rn")


def check_pairs(pairs, eps, D, kap_scale=1.0, model=None, expanded=False,
                form_scale=1.0):
    eps2 = pins.eps2_of(eps)
    # the set's largest squared norm, as the first screen kernel finds it
    Y = max(max(sq_norm64(x), sq_norm64(y)) for x, y in pairs)
    settled = {"in": 0, "out": 0, "exact": 0, "wrong": 0}
    for x, y in pairs:
        lo, hi = thresholds(sq_norm64(x), Y, eps2, D, kap_scale,
                            matrix=model is not None, expanded=expanded,
                            form_scale=form_scale)
        if model is None:
            v = screen_value(x, y)
        else:
            v = np.float32(float(matrix_screen_value(x, y, D, *model)))
        if expanded:
            exact = pins.exact_expanded_rounded(x, y) <= eps2
        else:
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


# The screen on the matrix cores (widths 16 and up): its thresholds are
# widened for an unspecified summation order, rounding and product rounding.
MATRIX_CASES = [(16, 3.0, 0.2), (20, 1.0, 0.3), (32, 1.0, 0.3), (48, 2.0, 0.5),
                (64, 1.0, 0.35), (64, 30.0, 1.0)]
MODELS = [("rn", True, "seq"), ("rn", False, "tree"), ("rz", False, "rev"),
          ("ru", False, "seq"), ("rd", True, "wide"), ("rd", False, "tree")]


@pytest.mark.parametrize("d,scale,eps", MATRIX_CASES)
def test_matrix_screen_decisions_agree_with_the_exact_distance(d, scale, eps):
    rng = np.random.default_rng(7000 + 1000 * d + int(scale))
    pairs = near_radius_pairs(rng, d, scale, eps, 60)
    for model in MODELS:
        settled = check_pairs(pairs, eps, compiled_width(d), model=model)
        assert settled["wrong"] == 0, (model, settled)
        if scale <= 3.0:
            assert settled["in"] > 1 and settled["out"] > 0, (model, settled)


def test_matrix_bound_without_the_rounding_terms_is_caught():
    wrong = 0
    for d, scale, eps in MATRIX_CASES:
        rng = np.random.default_rng(7000 + 1000 * d + int(scale))
        pairs = near_radius_pairs(rng, d, scale, eps, 60)
        for model in MODELS:
            wrong += check_pairs(pairs, eps, compiled_width(d), kap_scale=0.0,
                                 model=model)["wrong"]
    assert wrong > 0


# The hoisted-norm form as the decision (DBSCAN_FLAG_EXPANDED): the same
# screen values against thresholds that bracket that form's own exact
# decision, which differs from the direct one near the radius.
EXPANDED_CASES = [(1, 1.0, 0.01), (3, 1.0, 0.003), (3, 100.0, 0.05),
                  (3, 1e4, 2.0), (8, 1.0, 0.05), (16, 3.0, 0.2), (64, 1.0, 0.35),
                  (64, 30.0, 1.0)]


@pytest.mark.parametrize("d,scale,eps", EXPANDED_CASES)
def test_expanded_form_decisions(d, scale, eps):
    rng = np.random.default_rng(9000 + 1000 * d + int(scale))
    pairs = near_radius_pairs(rng, d, scale, eps, 150 if d < 32 else 60)
    D = compiled_width(d)
    models = [None] if D < 16 else [("rn", True, "seq"), ("rz", False, "rev"),
                                    ("rd", False, "tree")]
    for model in models:
        settled = check_pairs(pairs, eps, D, model=model, expanded=True)
        assert settled["wrong"] == 0, (model, settled)
        assert settled["exact"] > 0, (model, settled)
        if scale <= 3.0:
            assert settled["in"] > 1 and settled["out"] > 0, (model, settled)


def test_expanded_bound_without_rounding_terms_is_caught():
    """Thresholds with neither the screen's nor the form's rounding term
    settle some pair the wrong way, so the pairs do probe the bracket.
    (Dropping only the form's term is not caught here: on these pairs the
    screen's own worst-case term already covers the form's actual error.)"""
    wrong = 0
    for d, scale, eps in EXPANDED_CASES:
        rng = np.random.default_rng(9000 + 1000 * d + int(scale))
        pairs = near_radius_pairs(rng, d, scale, eps, 150 if d < 32 else 60)
        wrong += check_pairs(pairs, eps, compiled_width(d), kap_scale=0.0,
                             expanded=True, form_scale=0.0)["wrong"]
    assert wrong > 0
