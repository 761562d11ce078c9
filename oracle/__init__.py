"""ctypes front end of the brute-force DBSCAN oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the GPU library
never does, and has no fallback to it.  It shares no code with the GPU
path: inputs come from the seeded generators and results are compared
outside both.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# No -ffast-math, no FMA contraction: each operation of the distance is
# rounded on its own.  x86-64-v3 (AVX2) runs on any recent EPYC or Xeon.
CFLAGS = ["-O3", "-std=c11", "-march=x86-64-v3", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]

OK, BAD_ARG, NONFINITE, NO_MEMORY, FTZ_SET = 0, -1, -2, -4, -7

# Which distance decides "within eps" (oracle.h): the direct fp32 sum of
# squared differences, or the hoisted-norm form T + P - sum 2 x_k y_k.
FORMS = {"direct": 0, "expanded": 1}


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status}")
        self.status = status


def build(force: bool = False, out: str | None = None, src: str | None = None,
          extra: list[str] | None = None) -> str:
    """Compile oracle.c (or ``src``) into a shared library; returns its path."""
    src = src or _SRC
    out = out or _LIB
    if (not force and os.path.exists(out)
            and os.path.getmtime(out) >= os.path.getmtime(src)):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *(extra or []), "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True, cwd=os.path.dirname(src))
    os.replace(tmp, out)
    return out


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str | None = None):
        path = path or build()
        lib = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_d2.argtypes = [f32p, f32p, ctypes.c_int32]
        lib.oracle_d2.restype = ctypes.c_float
        lib.oracle_sq_norm.argtypes = [f32p, ctypes.c_int32]
        lib.oracle_sq_norm.restype = ctypes.c_float
        lib.oracle_d2_expanded.argtypes = [f32p, f32p, ctypes.c_int32]
        lib.oracle_d2_expanded.restype = ctypes.c_float
        lib.oracle_eps2.argtypes = [ctypes.c_float]
        lib.oracle_eps2.restype = ctypes.c_float
        lib.oracle_fit.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_float, ctypes.c_int32, i32p, i32p,
                                   ctypes.c_int32]
        lib.oracle_fit.restype = ctypes.c_int
        lib.oracle_fit_form.argtypes = lib.oracle_fit.argtypes + [ctypes.c_int32]
        lib.oracle_fit_form.restype = ctypes.c_int
        lib.oracle_row_counts.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_float, i64p, ctypes.c_int64,
                                          i32p, ctypes.c_int32]
        lib.oracle_row_counts.restype = ctypes.c_int
        lib.oracle_row_counts_form.argtypes = (lib.oracle_row_counts.argtypes
                                               + [ctypes.c_int32])
        lib.oracle_row_counts_form.restype = ctypes.c_int
        lib.oracle_row_neighbours.argtypes = [f32p, ctypes.c_int64,
                                              ctypes.c_int32, ctypes.c_float,
                                              ctypes.c_int64, i64p,
                                              ctypes.c_int64]
        lib.oracle_row_neighbours.restype = ctypes.c_int64
        lib.oracle_row_neighbours_form.argtypes = (
            lib.oracle_row_neighbours.argtypes + [ctypes.c_int32])
        lib.oracle_row_neighbours_form.restype = ctypes.c_int64
        lib.oracle_relabel.argtypes = [i32p, ctypes.c_int64, i32p, i32p]
        lib.oracle_relabel.restype = ctypes.c_int64
        lib.oracle_graph.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_float, i64p,
                                     ctypes.POINTER(i32p), ctypes.c_int32]
        lib.oracle_graph.restype = ctypes.c_int64
        lib.oracle_graph_form.argtypes = lib.oracle_graph.argtypes + [ctypes.c_int32]
        lib.oracle_graph_form.restype = ctypes.c_int64
        lib.oracle_free.argtypes = [ctypes.c_void_p]
        lib.oracle_free.restype = None
        lib.oracle_last_fit_seconds.argtypes = []
        lib.oracle_last_fit_seconds.restype = ctypes.c_double
        self.lib = lib
        self.path = path

    @staticmethod
    def _pts(points):
        x = np.ascontiguousarray(points, dtype=np.float32)
        if x.ndim == 1:
            x = x.reshape(-1, 1)
        return x

    def d2(self, a, b) -> np.float32:
        a = np.ascontiguousarray(a, dtype=np.float32).ravel()
        b = np.ascontiguousarray(b, dtype=np.float32).ravel()
        assert a.shape == b.shape
        f32p = ctypes.POINTER(ctypes.c_float)
        return np.float32(self.lib.oracle_d2(a.ctypes.data_as(f32p),
                                             b.ctypes.data_as(f32p), a.size))

    def d2_expanded(self, a, b) -> np.float32:
        """The hoisted-norm distance of two points (norms computed here)."""
        a = np.ascontiguousarray(a, dtype=np.float32).ravel()
        b = np.ascontiguousarray(b, dtype=np.float32).ravel()
        assert a.shape == b.shape
        f32p = ctypes.POINTER(ctypes.c_float)
        return np.float32(self.lib.oracle_d2_expanded(
            a.ctypes.data_as(f32p), b.ctypes.data_as(f32p), a.size))

    def sq_norm(self, a) -> np.float32:
        a = np.ascontiguousarray(a, dtype=np.float32).ravel()
        return np.float32(self.lib.oracle_sq_norm(
            a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), a.size))

    def eps2(self, eps) -> np.float32:
        return np.float32(self.lib.oracle_eps2(float(np.float32(eps))))

    def fit(self, points, eps, min_pts, n_threads: int = 0,
            form: str = "direct"):
        """Returns (labels int32[N], counts int32[N], seconds)."""
        x = self._pts(points)
        n, d = x.shape
        labels = np.empty(n, dtype=np.int32)
        counts = np.empty(n, dtype=np.int32)
        st = self.lib.oracle_fit_form(
            x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n, d,
            float(np.float32(eps)), int(min_pts),
            labels.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            counts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            int(n_threads), FORMS[form])
        if st != OK:
            raise OracleError(st)
        return labels, counts, self.lib.oracle_last_fit_seconds()

    def fit_status(self, points, n, d, eps, min_pts) -> int:
        """Raw status of a fit on possibly invalid arguments."""
        x = None if points is None else np.ascontiguousarray(points, np.float32)
        labels = np.empty(max(int(n), 1), dtype=np.int32)
        ptr = (None if x is None
               else x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        return self.lib.oracle_fit(ptr, int(n), int(d), float(np.float32(eps)),
                                   int(min_pts),
                                   labels.ctypes.data_as(
                                       ctypes.POINTER(ctypes.c_int32)),
                                   None, 1)

    def relabel(self, labels):
        """Returns (contiguous ids int32[N], sizes int32[K], K)."""
        lab = np.ascontiguousarray(labels, dtype=np.int32)
        n = lab.size
        out = np.empty(n, dtype=np.int32)
        sizes = np.empty(max(n, 1), dtype=np.int32)
        p = ctypes.POINTER(ctypes.c_int32)
        k = self.lib.oracle_relabel(lab.ctypes.data_as(p), n,
                                    out.ctypes.data_as(p),
                                    sizes.ctypes.data_as(p))
        if k < 0:
            raise OracleError(int(k))
        return out, sizes[:k].copy(), int(k)

    def graph(self, points, eps, n_threads: int = 0, form: str = "direct"):
        """Sparse eps-graph: (row_ptr int64[n+1], col_idx int32[nnz])."""
        x = self._pts(points)
        n, d = x.shape
        row_ptr = np.zeros(n + 1, dtype=np.int64)
        i32p = ctypes.POINTER(ctypes.c_int32)
        col = i32p()
        nnz = self.lib.oracle_graph_form(
            x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n, d,
            float(np.float32(eps)),
            row_ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            ctypes.byref(col), int(n_threads), FORMS[form])
        if nnz < 0:
            raise OracleError(int(nnz))
        try:
            col_idx = (np.ctypeslib.as_array(col, shape=(nnz,)).copy()
                       if nnz > 0 else np.zeros(0, dtype=np.int32))
        finally:
            self.lib.oracle_free(col)
        return row_ptr, col_idx

    def row_counts(self, points, eps, rows, n_threads: int = 0,
                   form: str = "direct") -> np.ndarray:
        x = self._pts(points)
        n, d = x.shape
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty(rows.size, dtype=np.int32)
        st = self.lib.oracle_row_counts_form(
            x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n, d,
            float(np.float32(eps)),
            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size,
            out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(n_threads),
            FORMS[form])
        if st != OK:
            raise OracleError(st)
        return out

    def row_neighbours(self, points, eps, i, form: str = "direct") -> np.ndarray:
        x = self._pts(points)
        n, d = x.shape
        cap = 1024
        while True:
            out = np.empty(cap, dtype=np.int64)
            c = self.lib.oracle_row_neighbours_form(
                x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n, d,
                float(np.float32(eps)), int(i),
                out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), cap,
                FORMS[form])
            if c < 0:
                raise OracleError(int(c))
            if c <= cap:
                return out[:c].copy()
            cap = int(c)


_default: Oracle | None = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
