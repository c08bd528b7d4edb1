"""ctypes binding of libnp.so (include/np.h): argument marshalling only.

Every step of the method runs in the HIP library; this module converts Python
arguments (NumPy arrays on the host, integer device pointers and stream
handles, e.g. torch's `tensor.data_ptr()` and `stream.cuda_stream`) into the
C ABI's plain pointers and sizes, and turns error codes into exceptions. It
raises at import time of the library if libnp.so has not been built; there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from functools import lru_cache

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnp.so")

NP_OK, NP_EINVAL, NP_ECAPACITY, NP_ENOMEM, NP_EHIP, NP_ESTATE, NP_EDEVICE = range(7)
MASK_UNION, MASK_INTERSECT, MASK_SINGLE = 0, 1, 2
MODES = {"union": MASK_UNION, "intersect": MASK_INTERSECT, "single": MASK_SINGLE}
ACT_RELU, ACT_SILU = 0, 1
REDUCE_ATOMIC, REDUCE_ORDERED = 0, 1
REDUCES = {"atomic": REDUCE_ATOMIC, "ordered": REDUCE_ORDERED}
LAYOUTS = {"slots": 0, "compact": 1}
ACTS = {"relu": ACT_RELU, "silu": ACT_SILU}
_NAMES = {0: "NP_OK", 1: "NP_EINVAL", 2: "NP_ECAPACITY", 3: "NP_ENOMEM", 4: "NP_EHIP",
          5: "NP_ESTATE", 6: "NP_EDEVICE"}

# every symbol include/np.h declares
EXPORTS = ["np_layer_create", "np_layer_destroy", "np_layer_reset", "np_delta_assign",
           "np_scatter_rows", "np_sparse_ffn", "np_decode_step", "np_layer_read_state",
           "np_layer_read_rows", "np_layer_info", "np_layer_counters", "np_layer_set_ffn_shape", "np_last_error",
           "np_layer_raise_error", "np_probe_read", "np_probe_read_set", "np_probe_copy", "np_decode_use_graphs", "np_layer_set_window",
           "np_sparse_ffn_acc", "np_layer_set_ffn_reduce", "np_layer_set_levels",
           "np_layer_set_layout", "np_layer_read_moves", "np_decode_set_staging",
           "np_layer_set_planar", "np_sparse_ffn_noalloc"]


class NPError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_NAMES.get(status, status)}: {msg}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("k_max", ctypes.c_int32),
                ("n_rows", ctypes.c_int32), ("n_centroids", ctypes.c_int32),
                ("mask_mode", ctypes.c_int32), ("act", ctypes.c_int32), ("device", ctypes.c_int32),
                ("masks", ctypes.c_void_p), ("row_store", ctypes.c_void_p)]


@lru_cache(maxsize=1)
def lib() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m delta_prefetched_ffn_amd.build` "
                           "(the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "np_layer_create": [ctypes.POINTER(LayerDesc), ctypes.POINTER(vp)],
        "np_layer_destroy": [vp],
        "np_layer_reset": [vp],
        "np_delta_assign": [vp, i32, i32, vp],
        "np_scatter_rows": [vp, vp],
        "np_sparse_ffn": [vp, vp, vp, vp],
        "np_decode_step": [vp, i32, vp, vp, vp, vp, vp],
        "np_layer_read_state": [vp, vp, vp, vp, vp, vp, vp, vp],
        "np_layer_read_rows": [vp, vp, i32, vp],
        "np_layer_info": [vp, vp],
        "np_layer_counters": [vp, vp],
        "np_layer_set_ffn_shape": [vp, i32, i32, i32],
        "np_layer_raise_error": [vp, i32, vp],
        "np_probe_read": [vp, i64, vp, vp],
        "np_probe_read_set": [vp, i32, i64, i32, vp, vp],
        "np_probe_copy": [vp, vp, i64, vp],
        "np_decode_use_graphs": [i32],
        "np_layer_set_window": [vp, i32],
        "np_sparse_ffn_acc": [vp, vp, vp, vp],
        "np_layer_set_ffn_reduce": [vp, i32],
        "np_layer_set_levels": [vp, i32, vp],
        "np_layer_set_layout": [vp, i32],
        "np_layer_read_moves": [vp, vp, vp, vp],
        "np_decode_set_staging": [i64, i32],
        "np_layer_set_planar": [vp, i32],
        "np_sparse_ffn_noalloc": [vp, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.np_last_error.argtypes = []
    L.np_last_error.restype = ctypes.c_char_p
    return L


def _check(status: int) -> None:
    if status != NP_OK:
        raise NPError(status, lib().np_last_error().decode())


def _ptr(a: np.ndarray | None) -> int | None:
    return None if a is None else a.ctypes.data


class Layer:
    """One sparse FFN layer (np_layer). row_store is a device or pinned-host pointer (int)."""

    def __init__(self, *, d_model: int, d_ff: int, k_max: int, n_rows: int, masks: np.ndarray,
                 mask_mode: int, row_store: int, device: int = 0, act: int = ACT_RELU,
                 keepalive=None):
        masks = np.ascontiguousarray(masks, dtype=np.uint64)
        n_tables = 1 if mask_mode == MASK_SINGLE else 2
        W = (d_ff + 63) // 64
        assert masks.ndim == 3 and masks.shape[0] == n_tables and masks.shape[2] == W, masks.shape
        desc = LayerDesc(d_model, d_ff, k_max, n_rows, masks.shape[1], mask_mode, act, device,
                         masks.ctypes.data, row_store)
        h = ctypes.c_void_p()
        _check(lib().np_layer_create(ctypes.byref(desc), ctypes.byref(h)))
        self.h = h
        self.d_model, self.d_ff, self.k_max, self.n_rows = d_model, d_ff, k_max, n_rows
        self._keepalive = keepalive

    def close(self) -> None:
        if self.h:
            _check(lib().np_layer_destroy(self.h))
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().np_layer_destroy(self.h)
        except Exception:
            pass

    def reset(self) -> None:
        _check(lib().np_layer_reset(self.h))

    def delta_assign(self, gate_cid: int, up_cid: int, stream: int = 0) -> None:
        _check(lib().np_delta_assign(self.h, gate_cid, up_cid, stream or None))

    def scatter_rows(self, stream: int = 0) -> None:
        _check(lib().np_scatter_rows(self.h, stream or None))

    def sparse_ffn(self, x_ptr: int, y_ptr: int, stream: int = 0) -> None:
        _check(lib().np_sparse_ffn(self.h, x_ptr, y_ptr, stream or None))

    def set_ffn_shape(self, slots_per_wg: int = 0, tile_cols: int = 0, threads: int = 0) -> None:
        _check(lib().np_layer_set_ffn_shape(self.h, slots_per_wg, tile_cols, threads))

    def sparse_ffn_acc(self, x_ptr: int, y_ptr: int, stream: int = 0) -> None:
        """y += FFN(x)."""
        _check(lib().np_sparse_ffn_acc(self.h, x_ptr, y_ptr, stream or None))

    def sparse_ffn_noalloc(self, x_ptr: int, y_ptr: int, stream: int = 0) -> None:
        """np_sparse_ffn_noalloc: the FFN with its exchange words in the library's static scratch."""
        _check(lib().np_sparse_ffn_noalloc(self.h, x_ptr, y_ptr, stream or None))

    def set_ffn_reduce(self, mode: str) -> None:
        """"ordered" (default; atomics-free, fixed order, bit-reproducible) or "atomic" (fp32 atomics, order free)."""
        _check(lib().np_layer_set_ffn_reduce(self.h, REDUCES[mode]))

    def set_window(self, window: int) -> None:
        """Residency window in tokens (1 = the buffer holds exactly the active set)."""
        _check(lib().np_layer_set_window(self.h, window))

    def set_levels(self, levels, n_levels: int) -> None:
        """Retention by frequency level: levels uint8 [d_ff], each < n_levels (0 switches it off)."""
        if n_levels == 0:
            _check(lib().np_layer_set_levels(self.h, 0, None))
            return
        lv = np.ascontiguousarray(levels, dtype=np.uint8)
        assert lv.shape == (self.d_ff,), lv.shape
        _check(lib().np_layer_set_levels(self.h, n_levels, lv.ctypes.data))

    def set_layout(self, layout: str) -> None:
        """"slots" (slot map, the default) or "compact" (active rows at positions 0 .. |S|-1)."""
        _check(lib().np_layer_set_layout(self.h, LAYOUTS[layout]))

    def set_planar(self, planar: bool) -> None:
        """Slot buffer as one plane per row kind (True) or one bundle per slot (False, the default)."""
        _check(lib().np_layer_set_planar(self.h, 1 if planar else 0))

    def raise_error(self, bits: int, stream: int = 0) -> None:
        """Raise device error bits as a failing kernel would (tests of error reporting)."""
        _check(lib().np_layer_raise_error(self.h, bits, stream or None))

    def read_moves(self) -> tuple[np.ndarray, np.ndarray]:
        """(src, dst) positions of the rows the last assignment moved (compact layout)."""
        src = np.empty(self.k_max, dtype=np.int32)
        dst = np.empty(self.k_max, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(lib().np_layer_read_moves(self.h, src.ctypes.data, dst.ctypes.data, ctypes.byref(n)))
        return src[: n.value].copy(), dst[: n.value].copy()

    def info(self) -> dict:
        out = np.zeros(6, dtype=np.int32)
        _check(lib().np_layer_info(self.h, out.ctypes.data))
        return dict(zip(["d_model", "d_ff", "k_max", "n_rows", "n_active", "n_in"], out.tolist()))

    def counters(self) -> tuple[int, int]:
        """(sum of |S|, sum of |D_in|) over accepted assignments since create/reset."""
        out = np.zeros(2, dtype=np.int64)
        _check(lib().np_layer_counters(self.h, out.ctypes.data))
        return int(out[0]), int(out[1])

    def read_state(self, check: bool = True) -> dict:
        K, M = self.k_max, self.d_ff
        st = {k: np.empty(K, dtype=np.int32) for k in ("owner", "d_in", "slot_in", "d_out", "act")}
        st["slot_map"] = np.empty(M, dtype=np.int32)
        counts = np.empty(4, dtype=np.int32)
        rc = lib().np_layer_read_state(self.h, _ptr(st["slot_map"]), _ptr(st["owner"]), _ptr(st["d_in"]),
                                       _ptr(st["slot_in"]), _ptr(st["d_out"]), _ptr(st["act"]),
                                       counts.ctypes.data)
        if check:
            _check(rc)
        n_in, n_out, n_act, err = counts.tolist()
        st["d_in"] = st["d_in"][:n_in]
        st["slot_in"] = st["slot_in"][:n_in]
        st["d_out"] = st["d_out"][:n_out]
        st["act"] = st["act"][:n_act]
        st["err"] = err
        return st

    def read_rows(self, slots=None) -> np.ndarray:
        """uint16 bf16 bits [n][n_rows][d_model]; slots=None reads the whole buffer."""
        if slots is None:
            out = np.empty((self.k_max, self.n_rows, self.d_model), dtype=np.uint16)
            _check(lib().np_layer_read_rows(self.h, None, self.k_max, out.ctypes.data))
            return out
        s = np.ascontiguousarray(slots, dtype=np.int32)
        out = np.empty((s.size, self.n_rows, self.d_model), dtype=np.uint16)
        _check(lib().np_layer_read_rows(self.h, s.ctypes.data, s.size, out.ctypes.data))
        return out


def decode_step(layers, cids: np.ndarray, x_ptr: int, y_ptr: int, compute_stream: int = 0,
                copy_stream: int | None = None) -> None:
    """np_decode_step over `layers` (list of Layer); cids int32 [n_layers][2] (host)."""
    cids = np.ascontiguousarray(cids, dtype=np.int32).reshape(len(layers), 2)
    handles = (ctypes.c_void_p * len(layers))(*[L.h.value for L in layers])
    cs = compute_stream or None
    ps = cs if copy_stream is None else (copy_stream or None)
    _check(lib().np_decode_step(handles, len(layers), cids.ctypes.data, x_ptr, y_ptr, cs, ps))


def decode_set_staging(nbytes: int, threads: int = 0) -> None:
    """Staged delta I/O for pinned host row stores (0 bytes: zero-copy pull, the default)."""
    _check(lib().np_decode_set_staging(nbytes, threads))


def decode_use_graphs(enable: bool) -> None:
    """np_decode_use_graphs: replay decode steps as captured HIP graphs, or launch one by one (default)."""
    _check(lib().np_decode_use_graphs(1 if enable else 0))


def probe_read(src_ptr: int, nbytes: int, sink_ptr: int, stream: int = 0) -> None:
    _check(lib().np_probe_read(src_ptr, nbytes, sink_ptr, stream or None))


def probe_read_set(src_ptrs, nbytes: int, passes: int, sink_ptr: int, stream: int = 0) -> None:
    arr = (ctypes.c_void_p * len(src_ptrs))(*src_ptrs)
    _check(lib().np_probe_read_set(arr, len(src_ptrs), nbytes, passes, sink_ptr, stream or None))


def probe_copy(dst_ptr: int, src_ptr: int, nbytes: int, stream: int = 0) -> None:
    _check(lib().np_probe_copy(dst_ptr, src_ptr, nbytes, stream or None))
