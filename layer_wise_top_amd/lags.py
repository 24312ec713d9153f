"""Python binding of liblags.so (include/lags.h): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels; torch provides
device memory and the current stream.  The functions keep the C names.  The
library must be built (``python -m layer_wise_top_amd.build``); loading it
without that raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblags.so")

LAGS_OK = 0
LAGS_ENOTINIT = -7
LAGS_ESTATIC = -8
LAGS_SPARSIFY_EXACT = 1
LAGS_MAX_LAYERS = 65536
LAGS_MAX_WORKERS = 1024

EXPORTED = (
    "lags_strerror", "lags_k_for_ratio", "lags_layout_create", "lags_layout_destroy",
    "lags_layout_num_elems", "lags_layout_total_k", "lags_layout_num_layers",
    "lags_layout_msg_offset", "lags_workspace_bytes", "lags_sparsify_layers",
    "lags_aggregate_apply", "lags_workspace_report", "lags_trace_enable",
    "lags_trace_read", "lags_num_kernels", "lags_kernel_name", "lags_sparsify_range",
    "lags_aggregate_range", "lags_merge_schedule", "lags_schedule_finish", "lags_adaptive_k",
    "lags_workspace_init", "lags_sparsify_layers_static",
)


class LagsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {strerror(status)} ({status})")
        self.status = status


class Report(ctypes.Structure):
    _fields_ = [("layers_sampled", ctypes.c_int32), ("layers_exact", ctypes.c_int32),
                ("bad_entries", ctypes.c_uint32), ("slow_chunks", ctypes.c_uint32),
                ("layers_wide_bin", ctypes.c_int32), ("fix_timeouts", ctypes.c_uint32)]


_lib = None


def lib():
    """Load liblags.so (raises if it has not been built).

    torch is imported first: its HIP runtime (torch/lib/libamdhip64.so, soname
    libamdhip64.so.7) must be the one the library binds to, since the device
    pointers and streams passed in come from torch.  Loaded the other way
    round, the library would pull the system runtime under its soname and
    torch would still load its own under the file name its libraries need:
    two runtimes in one process, the library's seeing no device."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m layer_wise_top_amd.build`")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, u32, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                             ctypes.c_void_p, ctypes.c_size_t)
    L.lags_strerror.restype = ctypes.c_char_p
    L.lags_strerror.argtypes = [ctypes.c_int]
    L.lags_k_for_ratio.restype = i64
    L.lags_k_for_ratio.argtypes = [i64, i64, i64]
    L.lags_layout_create.restype = ctypes.c_int
    L.lags_layout_create.argtypes = [i32, vp, vp, ctypes.POINTER(vp)]
    L.lags_layout_destroy.restype = None
    L.lags_layout_destroy.argtypes = [vp]
    for f in ("lags_layout_num_elems", "lags_layout_total_k"):
        getattr(L, f).restype = i64
        getattr(L, f).argtypes = [vp]
    L.lags_layout_num_layers.restype = i32
    L.lags_layout_num_layers.argtypes = [vp]
    L.lags_layout_msg_offset.restype = i64
    L.lags_layout_msg_offset.argtypes = [vp, i32]
    L.lags_workspace_bytes.restype = sz
    L.lags_workspace_bytes.argtypes = [vp, i32]
    L.lags_workspace_init.restype = ctypes.c_int
    L.lags_workspace_init.argtypes = [vp, vp, sz, i32, vp]
    L.lags_sparsify_layers.restype = ctypes.c_int
    L.lags_sparsify_layers.argtypes = [vp, vp, vp, vp, vp, vp, sz, u32, vp]
    L.lags_aggregate_apply.restype = ctypes.c_int
    L.lags_aggregate_apply.argtypes = [vp, vp, vp, vp, i32, ctypes.c_float, vp, sz, vp]
    L.lags_sparsify_layers_static.restype = ctypes.c_int
    L.lags_sparsify_layers_static.argtypes = [vp, vp, vp, vp, vp, u32, vp]
    L.lags_sparsify_range.restype = ctypes.c_int
    L.lags_sparsify_range.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, sz, u32, vp]
    L.lags_aggregate_range.restype = ctypes.c_int
    L.lags_aggregate_range.argtypes = [vp, i32, i32, vp, vp, vp, i32, ctypes.c_float, vp, sz, vp]
    f64 = ctypes.c_double
    L.lags_merge_schedule.restype = ctypes.c_int
    L.lags_merge_schedule.argtypes = [i32, vp, vp, f64, f64, vp, ctypes.POINTER(i32),
                                      ctypes.POINTER(f64)]
    L.lags_schedule_finish.restype = ctypes.c_int
    L.lags_schedule_finish.argtypes = [i32, vp, vp, f64, f64, vp, i32, ctypes.POINTER(f64)]
    L.lags_adaptive_k.restype = ctypes.c_int
    L.lags_adaptive_k.argtypes = [i32, vp, vp, i32, f64, f64, i64, i64, vp]
    L.lags_workspace_report.restype = ctypes.c_int
    L.lags_workspace_report.argtypes = [vp, vp, sz, vp, ctypes.POINTER(Report)]
    L.lags_trace_enable.restype = ctypes.c_int
    L.lags_trace_enable.argtypes = [vp, ctypes.c_int]
    L.lags_trace_read.restype = ctypes.c_int
    L.lags_trace_read.argtypes = [vp, vp, vp, i32]
    L.lags_num_kernels.restype = i32
    L.lags_num_kernels.argtypes = []
    L.lags_kernel_name.restype = ctypes.c_char_p
    L.lags_kernel_name.argtypes = [i32]
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().lags_strerror(int(status)).decode()


def _check(fn: str, rc: int):
    if rc != LAGS_OK:
        raise LagsError(fn, rc)


def lags_k_for_ratio(n: int, num: int, den: int) -> int:
    return int(lib().lags_k_for_ratio(int(n), int(num), int(den)))


def k_table(off, num, den) -> np.ndarray:
    """Per-layer k from exact ratios, through lags_k_for_ratio."""
    n = np.diff(np.asarray(off, np.int64))
    num = np.broadcast_to(np.asarray(num, np.int64), n.shape)
    den = np.broadcast_to(np.asarray(den, np.int64), n.shape)
    k = np.array([lags_k_for_ratio(a, b, c) for a, b, c in zip(n, num, den)], np.int64)
    if np.any(k < 0):
        raise ValueError("invalid ratio")
    return k


class Layout:
    """Owns one lags_layout (lags_layout_create / lags_layout_destroy)."""

    def __init__(self, off, k):
        off = np.ascontiguousarray(off, dtype=np.int64)
        k = np.ascontiguousarray(k, dtype=np.int64)
        if off.ndim != 1 or k.ndim != 1 or off.size != k.size + 1:
            raise ValueError("off must have L+1 entries and k L entries")
        h = ctypes.c_void_p()
        rc = lib().lags_layout_create(int(k.size), off.ctypes.data, k.ctypes.data, ctypes.byref(h))
        _check("lags_layout_create", rc)
        self._h = h
        self.off = off.copy()
        self.k = k.copy()
        self.L = int(lib().lags_layout_num_layers(h))
        self.n = int(lib().lags_layout_num_elems(h))
        self.K = int(lib().lags_layout_total_k(h))

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("layout destroyed")
        return self._h

    def msg_offset(self, l: int) -> int:
        return int(lib().lags_layout_msg_offset(self.handle, int(l)))

    def workspace_bytes(self, P: int = 1) -> int:
        return int(lib().lags_workspace_bytes(self.handle, int(P)))

    def close(self):
        if getattr(self, "_h", None) is not None:
            lib().lags_layout_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _dev_tensor(t, dtype, numel: int, name: str):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() < numel:
        raise ValueError(f"{name} must be contiguous with at least {numel} elements")
    return ctypes.c_void_p(t.data_ptr())


def workspace(layout: Layout, P: int = 1, device=None, stream=None):
    """Allocate a device workspace (uint8 tensor) for `layout` and up to P
    workers and initialise it (lags_workspace_init on `stream`, then that
    stream is synchronised, so the workspace is ready for calls on any
    stream)."""
    import torch
    nbytes = layout.workspace_bytes(P)
    if nbytes == 0:
        raise ValueError("invalid P")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
    lags_workspace_init(layout, ws, P, stream)
    (stream if stream is not None else torch.cuda.current_stream(ws.device)).synchronize()
    return ws


def lags_workspace_init(layout: Layout, ws, P: int = 1, stream=None):
    """Copy the layout's tables (and the chunk tables for P workers) into ws."""
    import torch
    w = _dev_tensor(ws, torch.uint8, 1, "ws")
    rc = lib().lags_workspace_init(layout.handle, w, ws.numel(), int(P), _stream_handle(stream))
    _check("lags_workspace_init", rc)


def lags_sparsify_layers(layout: Layout, grad, residual, msg_idx, msg_val, ws,
                         flags: int = 0, stream=None):
    import torch
    g = _dev_tensor(grad, torch.float32, layout.n, "grad")
    r = _dev_tensor(residual, torch.float32, layout.n, "residual")
    mi = _dev_tensor(msg_idx, torch.int32, layout.K, "msg_idx")  # uint32 bits
    mv = _dev_tensor(msg_val, torch.float32, layout.K, "msg_val")
    w = _dev_tensor(ws, torch.uint8, 1, "ws")
    rc = lib().lags_sparsify_layers(layout.handle, g, r, mi, mv, w, ws.numel(), int(flags),
                                    _stream_handle(stream))
    _check("lags_sparsify_layers", rc)


def lags_sparsify_layers_static(layout: Layout, grad, residual, msg_idx, msg_val, flags: int = 0,
                                stream=None):
    """lags_sparsify_layers on the library's static scratch (no workspace)."""
    import torch
    g = _dev_tensor(grad, torch.float32, layout.n, "grad")
    r = _dev_tensor(residual, torch.float32, layout.n, "residual")
    mi = _dev_tensor(msg_idx, torch.int32, layout.K, "msg_idx")
    mv = _dev_tensor(msg_val, torch.float32, layout.K, "msg_val")
    rc = lib().lags_sparsify_layers_static(layout.handle, g, r, mi, mv, int(flags),
                                           _stream_handle(stream))
    _check("lags_sparsify_layers_static", rc)


def lags_aggregate_apply(layout: Layout, weights, msg_idx, msg_val, P: int, lr: float, ws,
                         stream=None):
    import torch
    wt = _dev_tensor(weights, torch.float32, layout.n, "weights")
    mi = _dev_tensor(msg_idx, torch.int32, int(P) * layout.K, "msg_idx")
    mv = _dev_tensor(msg_val, torch.float32, int(P) * layout.K, "msg_val")
    w = _dev_tensor(ws, torch.uint8, 1, "ws")
    rc = lib().lags_aggregate_apply(layout.handle, wt, mi, mv, int(P), float(lr), w, ws.numel(),
                                    _stream_handle(stream))
    _check("lags_aggregate_apply", rc)


def lags_sparsify_range(layout: Layout, l0: int, l1: int, grad, residual, msg_idx, msg_val, ws,
                        flags: int = 0, stream=None):
    """Layers [l0, l1) only; the buffers are the full-model ones."""
    import torch
    g = _dev_tensor(grad, torch.float32, layout.n, "grad")
    r = _dev_tensor(residual, torch.float32, layout.n, "residual")
    mi = _dev_tensor(msg_idx, torch.int32, layout.K, "msg_idx")
    mv = _dev_tensor(msg_val, torch.float32, layout.K, "msg_val")
    w = _dev_tensor(ws, torch.uint8, 1, "ws")
    rc = lib().lags_sparsify_range(layout.handle, int(l0), int(l1), g, r, mi, mv, w, ws.numel(),
                                   int(flags), _stream_handle(stream))
    _check("lags_sparsify_range", rc)


def lags_aggregate_range(layout: Layout, l0: int, l1: int, weights, msg_idx, msg_val, P: int,
                         lr: float, ws, stream=None):
    """Layers [l0, l1) only; the buffers are the full-model ones."""
    import torch
    wt = _dev_tensor(weights, torch.float32, layout.n, "weights")
    mi = _dev_tensor(msg_idx, torch.int32, int(P) * layout.K, "msg_idx")
    mv = _dev_tensor(msg_val, torch.float32, int(P) * layout.K, "msg_val")
    w = _dev_tensor(ws, torch.uint8, 1, "ws")
    rc = lib().lags_aggregate_range(layout.handle, int(l0), int(l1), wt, mi, mv, int(P), float(lr),
                                    w, ws.numel(), _stream_handle(stream))
    _check("lags_aggregate_range", rc)


def lags_merge_schedule(backward_time, msg_bytes, alpha: float, beta: float):
    """Returns (runs, finish): runs is a list of (l0, l1) layer ranges in
    sending order (the first holds the last layer), finish the modelled time."""
    bt = np.ascontiguousarray(backward_time, dtype=np.float64)
    nb = np.ascontiguousarray(msg_bytes, dtype=np.int64)
    if bt.ndim != 1 or nb.shape != bt.shape:
        raise ValueError("backward_time and msg_bytes must be 1-D of one length")
    L = bt.size
    bounds = np.empty(L + 1, dtype=np.int32)
    nr = ctypes.c_int32()
    fin = ctypes.c_double()
    rc = lib().lags_merge_schedule(L, bt.ctypes.data, nb.ctypes.data, float(alpha), float(beta),
                                   bounds.ctypes.data, ctypes.byref(nr), ctypes.byref(fin))
    _check("lags_merge_schedule", rc)
    runs = [(int(bounds[j + 1]), int(bounds[j])) for j in range(nr.value)]
    return runs, fin.value


def lags_schedule_finish(backward_time, msg_bytes, alpha: float, beta: float, runs) -> float:
    """Modelled finish time of `runs` ((l0, l1) ranges in sending order)."""
    bt = np.ascontiguousarray(backward_time, dtype=np.float64)
    nb = np.ascontiguousarray(msg_bytes, dtype=np.int64)
    L = bt.size
    bounds = np.array([L] + [int(r[0]) for r in runs], dtype=np.int32)
    if any(int(r[1]) != int(bounds[j]) for j, r in enumerate(runs)):
        raise ValueError("runs are not consecutive in sending order")
    fin = ctypes.c_double()
    rc = lib().lags_schedule_finish(L, bt.ctypes.data, nb.ctypes.data, float(alpha), float(beta),
                                    bounds.ctypes.data, len(runs), ctypes.byref(fin))
    _check("lags_schedule_finish", rc)
    return fin.value


def lags_adaptive_k(off, backward_time, P: int, alpha: float, beta: float,
                    rmin=(1, 1000)) -> np.ndarray:
    """Per-layer k from each layer's overlap window (int64 [L])."""
    off = np.ascontiguousarray(off, dtype=np.int64)
    bt = np.ascontiguousarray(backward_time, dtype=np.float64)
    L = off.size - 1
    if bt.shape != (L,):
        raise ValueError("backward_time must have one entry per layer")
    k = np.empty(L, dtype=np.int64)
    rc = lib().lags_adaptive_k(L, off.ctypes.data, bt.ctypes.data, int(P), float(alpha),
                               float(beta), int(rmin[0]), int(rmin[1]), k.ctypes.data)
    _check("lags_adaptive_k", rc)
    return k


def lags_workspace_report(layout: Layout, ws, stream=None) -> dict:
    import torch
    w = _dev_tensor(ws, torch.uint8, 1, "ws")
    rep = Report()
    rc = lib().lags_workspace_report(layout.handle, w, ws.numel(), _stream_handle(stream),
                                     ctypes.byref(rep))
    _check("lags_workspace_report", rc)
    return {f: getattr(rep, f) for f, _ in Report._fields_}


def lags_trace_enable(layout: Layout, on: bool = True):
    _check("lags_trace_enable", lib().lags_trace_enable(layout.handle, 1 if on else 0))


def lags_trace_read(layout: Layout) -> dict:
    """{kernel name: (total ms, launches)} since tracing was enabled or last read."""
    nk = int(lib().lags_num_kernels())
    ms = (ctypes.c_double * nk)()
    cnt = (ctypes.c_int64 * nk)()
    _check("lags_trace_read", lib().lags_trace_read(layout.handle, ms, cnt, nk))
    return {lib().lags_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(nk)}


def kernel_names():
    return [lib().lags_kernel_name(i).decode() for i in range(int(lib().lags_num_kernels()))]
