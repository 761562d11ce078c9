"""Exact all-pairs DBSCAN on AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of
``libdbscan.so`` (``include/dbscan.h``).  This package binds that ABI with
ctypes (``_capi``: one function per C entry point) and adds ``fit``, which
takes torch tensors and uses torch only for device memory and the current
stream.  There is no CPU fallback.  The binding is loaded on first use, so
the seeded generators in ``datagen`` import without the library, and every
entry point raises ImportError when the library has not been built.
"""
from __future__ import annotations

import importlib

import numpy as np

_C_NAMES = {
    "FLAG_FORCE_TILE_MERGE", "FLAG_PRUNE_TILES", "FLAG_SCREEN",
    "FLAG_REVERSE_SCHEDULE", "FLAG_EXPANDED", "FLAG_SHUFFLE_SCHEDULE",
    "FLAG_TIME_PHASES", "MAX_D",
    "MERGE_EDGES",
    "MERGE_NONE", "MERGE_TILES", "dbscan_abi_version", "dbscan_fit",
    "dbscan_fit_counts", "dbscan_fit_device_noalloc", "ERR_TOO_LARGE",
    "NOALLOC_SCRATCH_BYTES",
    "dbscan_fit_device", "dbscan_fit_device_ex", "dbscan_info",
    "dbscan_status_string", "dbscan_workspace_bytes",
    "dbscan_workspace_bytes_with_edges", "dbscan_relabel_device",
    "dbscan_relabel_workspace_bytes", "dbscan_graph_device",
    "dbscan_graph_workspace_bytes", "ERR_CAPACITY", "ERR_WORKSPACE",
}


def _c():
    return importlib.import_module(__name__ + "._capi")


def __getattr__(name):
    if name in _C_NAMES:
        return getattr(_c(), name)
    raise AttributeError(name)


__all__ = [
    "DbscanError", "Workspace", "fit", "fit_host", "dbscan_fit",
    "dbscan_fit_counts", "dbscan_fit_device_noalloc",
    "dbscan_fit_device", "dbscan_fit_device_ex", "dbscan_workspace_bytes",
    "dbscan_workspace_bytes_with_edges", "dbscan_status_string",
    "dbscan_abi_version", "dbscan_info", "relabel",
    "dbscan_relabel_device", "dbscan_relabel_workspace_bytes", "graph",
    "dbscan_graph_device", "dbscan_graph_workspace_bytes",
]


class DbscanError(RuntimeError):
    def __init__(self, status: int, hip_error: int = 0):
        msg = f"dbscan status {status}: {_c().dbscan_status_string(status)}"
        if hip_error:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


def default_edge_capacity(device=None) -> int:
    """Edge-area size used when none is given: a quarter of the free device
    memory, at most 16 GiB (8 bytes per neighbour pair)."""
    import torch
    free, _ = torch.cuda.mem_get_info(device)
    return int(min(free // 4, 16 << 30) // 8)


class Workspace:
    """A reusable device workspace (torch uint8 tensor) for fits of up to
    ``n`` points of dimension ``d`` with room for ``max_edges`` pairs."""

    def __init__(self, n: int, d: int, max_edges: int | None = None,
                 device="cuda"):
        import torch
        if max_edges is None:
            max_edges = default_edge_capacity(device)
        nbytes = _c().dbscan_workspace_bytes_with_edges(n, d, max_edges)
        if nbytes == 0:
            raise DbscanError(_c().ERR_INVALID_ARG)
        self.n, self.d, self.max_edges = n, d, max_edges
        self.tensor = torch.empty(nbytes, dtype=torch.uint8, device=device)

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr()

    @property
    def nbytes(self) -> int:
        return self.tensor.numel()


def fit(x, eps: float, min_pts: int, *, return_counts: bool = False,
        workspace: Workspace | None = None, max_edges: int | None = None,
        flags: int = 0, return_info: bool = False, stream=None):
    """Cluster the rows of ``x`` (torch float32 [N, d], contiguous, on a
    gfx950 device).  Returns int32 labels on the device (-1 = noise; a
    cluster's label is its smallest point index), then the int32 neighbour
    counts if ``return_counts``, then a dict of ``dbscan_info`` fields if
    ``return_info``."""
    import torch
    c = _c()
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32:
        raise TypeError("x must be a torch.float32 tensor")
    if x.dim() == 1:
        x = x.reshape(-1, 1)
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [N, d] tensor on the GPU")
    n, d = x.shape
    labels = torch.empty(n, dtype=torch.int32, device=x.device)
    counts = (torch.empty(n, dtype=torch.int32, device=x.device)
              if return_counts else None)
    if workspace is None:
        workspace = Workspace(n, d, max_edges, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    info = c.dbscan_info()
    st = c.dbscan_fit_device_ex(
        x.data_ptr() if n else None, n, d, float(eps), int(min_pts),
        labels.data_ptr() if n else None,
        counts.data_ptr() if (counts is not None and n) else None,
        workspace.ptr, workspace.nbytes, stream.cuda_stream, int(flags), info)
    if st != 0:
        raise DbscanError(st, info.hip_error)
    out = [labels]
    if return_counts:
        out.append(counts)
    if return_info:
        out.append(info.as_dict())
    return out[0] if len(out) == 1 else tuple(out)


def graph(x, eps: float, *, max_pairs: int | None = None, flags: int = 0,
          return_info: bool = False, stream=None):
    """Sparse eps-graph of the rows of ``x`` (torch float32 [N, d] on the
    GPU) in CSR form: returns int64 ``row_ptr`` [N+1] and int32 ``col_idx``
    [nnz] on the device; row i lists every j with d2(i, j) <= eps^2, i
    itself included, in ascending j.  ``max_pairs`` sizes the first attempt
    (neighbour pairs i<j); when the graph is larger the call is repeated
    once with the sizes the library reported."""
    import ctypes
    import torch
    c = _c()
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32:
        raise TypeError("x must be a torch.float32 tensor")
    if x.dim() == 1:
        x = x.reshape(-1, 1)
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [N, d] tensor on the GPU")
    n, d = x.shape
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    if max_pairs is None:
        max_pairs = min(64 * n, default_edge_capacity(x.device))
    row_ptr = torch.empty(n + 1, dtype=torch.int64, device=x.device)
    for attempt in range(2):
        nbytes = c.dbscan_graph_workspace_bytes(n, d, max_pairs)
        if nbytes == 0:
            raise DbscanError(c.ERR_INVALID_ARG)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
        col = torch.empty(max(n + 2 * max_pairs, 1), dtype=torch.int32,
                          device=x.device)
        nnz = ctypes.c_int64(0)
        info = c.dbscan_info()
        st = c.dbscan_graph_device(
            x.data_ptr() if n else None, n, d, float(eps), row_ptr.data_ptr(),
            col.data_ptr(), col.numel(), nnz, ws.data_ptr(), ws.numel(),
            stream.cuda_stream, int(flags), info)
        if attempt == 0 and st in (c.ERR_CAPACITY, c.ERR_WORKSPACE):
            max_pairs = int(info.n_edges)
            del ws, col
            continue
        break
    if st != 0:
        raise DbscanError(st, info.hip_error)
    out = (row_ptr, col[:nnz.value])
    return out + (info.as_dict(),) if return_info else out


def relabel(labels, return_sizes: bool = True, stream=None):
    """Contiguous cluster ids 0..K-1 (ascending smallest member; noise -1)
    for int32 device labels from ``fit``.  Returns ids, and the int32 sizes
    of the K clusters if ``return_sizes``."""
    import ctypes
    import torch
    c = _c()
    if labels.dtype != torch.int32 or not labels.is_cuda:
        raise TypeError("labels must be int32 on the GPU")
    labels = labels.contiguous()
    n = labels.numel()
    ids = torch.empty_like(labels)
    sizes = torch.empty(max(n, 1), dtype=torch.int32, device=labels.device)
    ws = torch.empty(c.dbscan_relabel_workspace_bytes(n), dtype=torch.uint8,
                     device=labels.device)
    k = ctypes.c_int64(0)
    if stream is None:
        stream = torch.cuda.current_stream(labels.device)
    st = c.dbscan_relabel_device(
        labels.data_ptr() if n else None, n, ids.data_ptr() if n else None,
        sizes.data_ptr() if return_sizes else None, k, ws.data_ptr(),
        ws.numel(), stream.cuda_stream)
    if st != 0:
        raise DbscanError(st)
    return (ids, sizes[:k.value]) if return_sizes else ids


def fit_host(points, eps: float, min_pts: int, return_counts: bool = False):
    """Host arrays in and out through the allocating C entries
    ``dbscan_fit`` (labels) and ``dbscan_fit_counts`` (labels and counts)."""
    x = np.ascontiguousarray(points, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(-1, 1)
    n, d = x.shape
    labels = np.empty(n, dtype=np.int32)
    counts = np.empty(n, dtype=np.int32) if return_counts else None
    if counts is None:
        st = _c().dbscan_fit(x.ctypes.data if n else None, n, d, float(eps),
                             int(min_pts), labels.ctypes.data if n else None)
    else:
        st = _c().dbscan_fit_counts(
            x.ctypes.data if n else None, n, d, float(eps), int(min_pts),
            labels.ctypes.data if n else None, counts.ctypes.data if n else None)
    if st != 0:
        raise DbscanError(st)
    return (labels, counts) if return_counts else labels
