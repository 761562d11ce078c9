"""Seeded synthetic point sets for the DBSCAN engine and its tests.

This module draws random inputs and nothing else: it holds no distance,
neighbourhood or clustering arithmetic, so the GPU path and the CPU
oracle can both be fed from it without sharing any of the method.

Reproducibility rules (the same bytes on every x86-64 host with this
numpy): values come from ``numpy.random.Generator(PCG64(seed))`` in
float64 and are built only from +, -, *, / and sqrt, which IEEE 754 rounds
correctly everywhere.  No numpy transcendental ufunc and no BLAS/LAPACK
call is used, because those dispatch to CPU-specific code paths whose last
bits may differ between machines.  Directions on circles and spheres are
normalised Gaussian vectors; the orthonormal embedding of the 64-d set is
a modified Gram-Schmidt in plain Python floats.  Every set is cast to
float32 and then shuffled with ``rng.permutation`` so that point index
order does not follow the cluster structure.

The five named workloads stand in for the point sets that the CUDA DBSCAN
paper (Wang et al., "Design and optimization of DBSCAN Algorithm based on
CUDA", Sec. V, Tables III-V: an unnamed 3-D set of 5,061 to 60,032 points)
and the PyRKNN summary (Embed200: low-dimensional Gaussian blobs embedded
in a high-dimensional space plus uniform noise) measure on; none of those
data sets is reproduced.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_workload",
    "sha256_points",
    "uniform_points",
    "gaussian_blobs",
    "integer_lattice",
    "collinear_chain",
]


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    n: int
    d: int
    eps: float
    min_pts: int
    recipe: str


WORKLOADS = {
    1: Workload(1, "blobs2d_n2000", 2000, 2, 0.03, 5,
                "5 Gaussian blobs (centres U[0,1]^2, sigma 0.05, 360 points "
                "each) + 200 U[0,1]^2 noise points"),
    2: Workload(2, "blobs_rings2d_n50000", 50000, 2, 0.01, 10,
                "20 Gaussian blobs x 1500 (centres U[0,1]^2, sigma "
                "U[0.005,0.02]) + rings about (0.5,0.5): 6000 at r=0.3 and "
                "9000 at r=0.45, radial sigma 0.005 + 5000 U[0,1]^2 noise"),
    3: Workload(3, "zipf_blobs8d_n200000", 200000, 8, 0.05, 20,
                "50 Gaussian blobs in [0,1]^8 (sigma U[0.01,0.04]), sizes "
                "proportional to rank^-1.2 rounded by largest remainder to "
                "190000 + 10000 U[0,1]^8 noise"),
    4: Workload(4, "blobs_walks3d_n1000000", 1000000, 3, 0.003, 16,
                "200 Gaussian blobs x 2250 (centres U[0,1]^3, sigma 0.004) + "
                "100 random walks x 4500 (start U[0,1]^3, step 0.001 in a "
                "uniform random direction) + 100000 U[0,1]^3 noise"),
    5: Workload(5, "embedded_blobs64d_n262144", 262144, 64, 0.35, 10,
                "32 Gaussian blobs (7782 or 7783 points) in a 6-d latent "
                "space (centres U[-1,1]^6, sigma 0.1) mapped to 64-d by a "
                "seeded orthonormal 6x64 map, + iid N(0,0.01^2) per "
                "coordinate; + 13107 U[-1,1]^64 noise"),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _finish(parts, rng) -> np.ndarray:
    x = np.concatenate(parts, axis=0).astype(np.float32)
    perm = rng.permutation(x.shape[0])
    return np.ascontiguousarray(x[perm])


def _sum_sq_rows(g: np.ndarray) -> np.ndarray:
    # explicit left-to-right column sum (no pairwise/SIMD reduction order)
    acc = g[:, 0] * g[:, 0]
    for k in range(1, g.shape[1]):
        acc = acc + g[:, k] * g[:, k]
    return acc


def _unit_dirs_exact(rng, count: int, dim: int) -> np.ndarray:
    g = rng.standard_normal((count, dim))
    norm = np.sqrt(_sum_sq_rows(g))
    norm[norm == 0.0] = 1.0
    return g / norm[:, None]


def _w1(rng):
    centres = rng.uniform(0.0, 1.0, (5, 2))
    parts = [c + 0.05 * rng.standard_normal((360, 2)) for c in centres]
    parts.append(rng.uniform(0.0, 1.0, (200, 2)))
    return _finish(parts, rng)


def _w2(rng):
    parts = []
    centres = rng.uniform(0.0, 1.0, (20, 2))
    sigmas = rng.uniform(0.005, 0.02, 20)
    for c, s in zip(centres, sigmas):
        parts.append(c + s * rng.standard_normal((1500, 2)))
    for radius, count in ((0.3, 6000), (0.45, 9000)):
        dirs = _unit_dirs_exact(rng, count, 2)
        r = radius + 0.005 * rng.standard_normal(count)
        parts.append(0.5 + r[:, None] * dirs)
    parts.append(rng.uniform(0.0, 1.0, (5000, 2)))
    return _finish(parts, rng)


def zipf_sizes(count: int, total: int, s: float) -> list[int]:
    """Integer sizes proportional to rank^-s (rank 1..count) that sum to
    ``total``, by largest-remainder rounding (ties to the lower rank)."""
    w = [float(r) ** (-s) for r in range(1, count + 1)]
    wsum = math.fsum(w)
    exact = [total * wi / wsum for wi in w]
    base = [int(math.floor(e)) for e in exact]
    rem = total - sum(base)
    order = sorted(range(count), key=lambda i: (-(exact[i] - base[i]), i))
    for i in order[:rem]:
        base[i] += 1
    return base


def _w3(rng):
    sizes = zipf_sizes(50, 190000, 1.2)
    centres = rng.uniform(0.0, 1.0, (50, 8))
    sigmas = rng.uniform(0.01, 0.04, 50)
    parts = [c + s * rng.standard_normal((m, 8))
             for c, s, m in zip(centres, sigmas, sizes)]
    parts.append(rng.uniform(0.0, 1.0, (10000, 8)))
    return _finish(parts, rng)


def _w4(rng):
    parts = []
    centres = rng.uniform(0.0, 1.0, (200, 3))
    for c in centres:
        parts.append(c + 0.004 * rng.standard_normal((2250, 3)))
    starts = rng.uniform(0.0, 1.0, (100, 3))
    for s0 in starts:
        steps = 0.001 * _unit_dirs_exact(rng, 4499, 3)
        walk = np.empty((4500, 3))
        walk[0] = s0
        walk[1:] = s0 + np.cumsum(steps, axis=0)
        parts.append(walk)
    parts.append(rng.uniform(0.0, 1.0, (100000, 3)))
    return _finish(parts, rng)


def orthonormal_rows(rng, rows: int, cols: int) -> np.ndarray:
    """``rows`` orthonormal vectors of length ``cols``: modified Gram-Schmidt
    of the columns of a seeded cols x rows standard-normal matrix, done in
    plain Python floats so the result does not depend on a BLAS build."""
    a = rng.standard_normal((cols, rows))
    vecs = [[float(a[i, j]) for i in range(cols)] for j in range(rows)]
    out = []
    for v in vecs:
        w = list(v)
        for q in out:
            dot = 0.0
            for i in range(cols):
                dot += q[i] * w[i]
            w = [w[i] - dot * q[i] for i in range(cols)]
        nrm = 0.0
        for i in range(cols):
            nrm += w[i] * w[i]
        nrm = math.sqrt(nrm)
        out.append([wi / nrm for wi in w])
    return np.array(out, dtype=np.float64)


def _w5(rng):
    n_noise = 13107
    n_blob = 262144 - n_noise
    base, extra = divmod(n_blob, 32)
    sizes = [base + (1 if b < extra else 0) for b in range(32)]
    m = orthonormal_rows(rng, 6, 64)           # 6 x 64
    centres = rng.uniform(-1.0, 1.0, (32, 6))
    parts = []
    for c, size in zip(centres, sizes):
        z = c + 0.1 * rng.standard_normal((size, 6))
        x = z[:, 0:1] * m[0]
        for k in range(1, 6):
            x = x + z[:, k:k + 1] * m[k]
        parts.append(x + 0.01 * rng.standard_normal((size, 64)))
    parts.append(rng.uniform(-1.0, 1.0, (n_noise, 64)))
    return _finish(parts, rng)


_BUILDERS = {1: _w1, 2: _w2, 3: _w3, 4: _w4, 5: _w5}


def make_workload(key: int):
    """Return ``(points float32 [N, d] C-contiguous, eps, min_pts, Workload)``
    for workload ``key`` in 1..5 (seed 1000 + key)."""
    w = WORKLOADS[key]
    x = _BUILDERS[key](_rng(1000 + key))
    assert x.shape == (w.n, w.d) and x.dtype == np.float32
    return x, w.eps, w.min_pts, w


def sha256_points(x: np.ndarray) -> str:
    a = np.ascontiguousarray(x, dtype=np.float32)
    return hashlib.sha256(a.tobytes()).hexdigest()


# ---------------------------------------------------------------- test shapes

def uniform_points(n: int, d: int, seed: int, lo: float = 0.0,
                   hi: float = 1.0) -> np.ndarray:
    rng = _rng(seed)
    return np.ascontiguousarray(rng.uniform(lo, hi, (n, d)).astype(np.float32))


def gaussian_blobs(n: int, d: int, seed: int, n_blobs: int = 4,
                   sigma: float = 0.05, noise_frac: float = 0.1) -> np.ndarray:
    """Blobs with centres U[0,1]^d plus uniform noise, shuffled."""
    rng = _rng(seed)
    n_noise = int(n * noise_frac)
    n_b = n - n_noise
    centres = rng.uniform(0.0, 1.0, (max(n_blobs, 1), d))
    labels = rng.integers(0, max(n_blobs, 1), n_b)
    pts = centres[labels] + sigma * rng.standard_normal((n_b, d))
    parts = [pts, rng.uniform(0.0, 1.0, (n_noise, d))]
    return _finish(parts, rng)


def integer_lattice(side: int, d: int) -> np.ndarray:
    """All points of {0..side-1}^d, row-major (last coordinate fastest)."""
    grids = np.meshgrid(*([np.arange(side)] * d), indexing="ij")
    pts = np.stack([g.reshape(-1) for g in grids[::-1]], axis=1)
    return np.ascontiguousarray(pts.astype(np.float32))


def collinear_chain(n: int, step: float, d: int = 1) -> np.ndarray:
    """Points k*step (float32 of the float64 product) on the first axis."""
    x = np.zeros((n, d), dtype=np.float64)
    x[:, 0] = np.arange(n, dtype=np.float64) * step
    return np.ascontiguousarray(x.astype(np.float32))
