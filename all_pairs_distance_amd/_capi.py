"""ctypes binding of libdbscan.so, one Python function per C entry point
(same names, same arguments).  Argument marshalling only: every step of a
fit runs in the library's HIP kernels.  There is no CPU fallback: if the
library is missing, importing this module raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdbscan.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "dbscan.h")

OK = 0
ERR_INVALID_ARG = -1
ERR_NONFINITE = -2
ERR_NO_DEVICE = -3
ERR_OOM = -4
ERR_WORKSPACE = -5
ERR_HIP = -6
ERR_CAPACITY = -7
ERR_TOO_LARGE = -8
NOALLOC_SCRATCH_BYTES = 64 << 20

MERGE_NONE, MERGE_EDGES, MERGE_TILES = 0, 1, 2
FLAG_TIME_PHASES = 0x1
FLAG_FORCE_TILE_MERGE = 0x2
FLAG_PRUNE_TILES = 0x4
FLAG_SCREEN = 0x8
FLAG_REVERSE_SCHEDULE = 0x10
FLAG_EXPANDED = 0x20
FLAG_SHUFFLE_SCHEDULE = 0x40
MAX_D = 64


class dbscan_info(ctypes.Structure):
    _fields_ = [
        ("n_core", ctypes.c_int64),
        ("n_edges", ctypes.c_int64),
        ("edge_capacity", ctypes.c_int64),
        ("pass1_pairs", ctypes.c_int64),
        ("pass2_pairs", ctypes.c_int64),
        ("tiles_total", ctypes.c_int64),
        ("tiles_kept", ctypes.c_int64),
        ("merge_mode", ctypes.c_int32),
        ("timed", ctypes.c_int32),
        ("ms_layout", ctypes.c_float),
        ("ms_count", ctypes.c_float),
        ("ms_core", ctypes.c_float),
        ("ms_merge", ctypes.c_float),
        ("ms_label", ctypes.c_float),
        ("ms_total", ctypes.c_float),
        ("hip_error", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


def _load() -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime (soname libamdhip64.so.7).  Load it
    # first so that this library binds to that same runtime: a second HIP /
    # HSA runtime in the process would not see the device, and torch's
    # device memory must be used through the runtime that allocated it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m all_pairs_distance_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.dbscan_workspace_bytes.argtypes = [i64, i32]
    lib.dbscan_workspace_bytes.restype = ctypes.c_size_t
    lib.dbscan_workspace_bytes_with_edges.argtypes = [i64, i32, i64]
    lib.dbscan_workspace_bytes_with_edges.restype = ctypes.c_size_t
    lib.dbscan_fit_device.argtypes = [vp, i64, i32, f32, i32, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.dbscan_fit_device.restype = ctypes.c_int
    lib.dbscan_fit_device_ex.argtypes = [vp, i64, i32, f32, i32, vp, vp, vp,
                                         ctypes.c_size_t, vp, ctypes.c_uint32,
                                         ctypes.POINTER(dbscan_info)]
    lib.dbscan_fit_device_ex.restype = ctypes.c_int
    lib.dbscan_fit_device_noalloc.argtypes = [vp, i64, i32, f32, i32, vp,
                                              vp, vp]
    lib.dbscan_fit_device_noalloc.restype = ctypes.c_int
    lib.dbscan_fit.argtypes = [vp, i64, i32, f32, i32, vp]
    lib.dbscan_fit.restype = ctypes.c_int
    lib.dbscan_fit_counts.argtypes = [vp, i64, i32, f32, i32, vp, vp]
    lib.dbscan_fit_counts.restype = ctypes.c_int
    lib.dbscan_relabel_workspace_bytes.argtypes = [i64]
    lib.dbscan_relabel_workspace_bytes.restype = ctypes.c_size_t
    lib.dbscan_relabel_device.argtypes = [vp, i64, vp, vp,
                                          ctypes.POINTER(ctypes.c_int64), vp,
                                          ctypes.c_size_t, vp]
    lib.dbscan_relabel_device.restype = ctypes.c_int
    lib.dbscan_graph_workspace_bytes.argtypes = [i64, i32, i64]
    lib.dbscan_graph_workspace_bytes.restype = ctypes.c_size_t
    lib.dbscan_graph_device.argtypes = [vp, i64, i32, f32, vp, vp, i64,
                                        ctypes.POINTER(ctypes.c_int64), vp,
                                        ctypes.c_size_t, vp, ctypes.c_uint32,
                                        ctypes.POINTER(dbscan_info)]
    lib.dbscan_graph_device.restype = ctypes.c_int
    lib.dbscan_status_string.argtypes = [ctypes.c_int]
    lib.dbscan_status_string.restype = ctypes.c_char_p
    lib.dbscan_abi_version.argtypes = []
    lib.dbscan_abi_version.restype = ctypes.c_int
    return lib


lib = _load()


def dbscan_workspace_bytes(n: int, d: int) -> int:
    return int(lib.dbscan_workspace_bytes(n, d))


def dbscan_workspace_bytes_with_edges(n: int, d: int, max_edges: int) -> int:
    return int(lib.dbscan_workspace_bytes_with_edges(n, d, max_edges))


def dbscan_fit_device(d_points: int, n: int, d: int, eps: float, min_pts: int,
                      d_labels: int, d_counts: int | None, d_workspace: int,
                      workspace_bytes: int, hip_stream: int | None) -> int:
    return int(lib.dbscan_fit_device(d_points, n, d, eps, min_pts, d_labels,
                                      d_counts, d_workspace, workspace_bytes,
                                      hip_stream))


def dbscan_fit_device_ex(d_points: int, n: int, d: int, eps: float,
                         min_pts: int, d_labels: int, d_counts: int | None,
                         d_workspace: int, workspace_bytes: int,
                         hip_stream: int | None, flags: int = 0,
                         info: dbscan_info | None = None) -> int:
    return int(lib.dbscan_fit_device_ex(
        d_points, n, d, eps, min_pts, d_labels, d_counts, d_workspace,
        workspace_bytes, hip_stream, flags,
        ctypes.byref(info) if info is not None else None))


def dbscan_fit_device_noalloc(d_points: int, n: int, d: int, eps: float,
                              min_pts: int, d_labels: int,
                              d_counts: int | None,
                              hip_stream: int | None) -> int:
    """Device-pointer fit in the library's fixed per-GPU scratch (no
    workspace, no allocation)."""
    return int(lib.dbscan_fit_device_noalloc(d_points, n, d, eps, min_pts,
                                             d_labels, d_counts, hip_stream))


def dbscan_fit(points: int, n: int, d: int, eps: float, min_pts: int,
               labels: int) -> int:
    """Host-pointer entry: points/labels are host addresses."""
    return int(lib.dbscan_fit(points, n, d, eps, min_pts, labels))


def dbscan_fit_counts(points: int, n: int, d: int, eps: float, min_pts: int,
                      labels: int, counts: int | None) -> int:
    """Host-pointer entry with neighbour counts (host address or None)."""
    return int(lib.dbscan_fit_counts(points, n, d, eps, min_pts, labels,
                                     counts))


def dbscan_relabel_workspace_bytes(n: int) -> int:
    return int(lib.dbscan_relabel_workspace_bytes(n))


def dbscan_relabel_device(d_labels: int, n: int, d_ids: int,
                          d_sizes: int | None, n_clusters, d_workspace: int,
                          workspace_bytes: int, hip_stream: int | None) -> int:
    """n_clusters: a ctypes.c_int64 (or None)."""
    return int(lib.dbscan_relabel_device(
        d_labels, n, d_ids, d_sizes,
        ctypes.byref(n_clusters) if n_clusters is not None else None,
        d_workspace, workspace_bytes, hip_stream))


def dbscan_graph_workspace_bytes(n: int, d: int, max_pairs: int) -> int:
    return int(lib.dbscan_graph_workspace_bytes(n, d, max_pairs))


def dbscan_graph_device(d_points: int, n: int, d: int, eps: float,
                        d_row_ptr: int, d_col_idx: int | None,
                        col_capacity: int, nnz_out, d_workspace: int,
                        workspace_bytes: int, hip_stream: int | None,
                        flags: int = 0, info: dbscan_info | None = None) -> int:
    """nnz_out: a ctypes.c_int64 (or None)."""
    return int(lib.dbscan_graph_device(
        d_points, n, d, eps, d_row_ptr, d_col_idx, col_capacity,
        ctypes.byref(nnz_out) if nnz_out is not None else None,
        d_workspace, workspace_bytes, hip_stream, flags,
        ctypes.byref(info) if info is not None else None))


def dbscan_status_string(status: int) -> str:
    return lib.dbscan_status_string(status).decode()


def dbscan_abi_version() -> int:
    return int(lib.dbscan_abi_version())
