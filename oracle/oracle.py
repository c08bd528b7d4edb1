"""Python access to the CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module. It shares no code with the HIP library.

The oracle follows "NeuroPrefetcher: Storage-Aware Sparse LLM Inference via
Delta Prefetching" (Dhar et al.), section 3.4 (active set from centroid
masks, delta by set difference, slot map with -1 for non-resident neurons,
freed slots reused without compaction, cold start) and section 3.5 (sorted
incoming IDs, neuron-centric [gate|up|down^T] records), with the readings
listed in oracle.c's header.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

UNION, INTERSECT, SINGLE = 0, 1, 2
MODES = {"union": UNION, "intersect": INTERSECT, "single": SINGLE}
RELU, SILU = 0, 1
ACTS = {"relu": RELU, "silu": SILU}
_OK, _EINVAL, _ECAPACITY = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build_lib(force: bool = False) -> str:
    """Compile oracle.c (gcc -O2, strict IEEE: no fast-math) into liboracle.so."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = f"gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -o {tmp} {src} -lm"
        if os.system(cmd) != 0:
            raise RuntimeError(f"failed: {cmd}")
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized_lib(out_dir: str, force: bool = False) -> str:
    """oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (clang, shared sanitizer
    runtime, any UB report fatal) into out_dir/liboracle_san.so, for the host sanitizer tests."""
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(out_dir, "liboracle_san.so")
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        os.makedirs(out_dir, exist_ok=True)
        tmp = out + f".tmp{os.getpid()}"
        cmd = (f"{SAN_CC} -O1 -g -std=c11 -fPIC -shared -ffp-contract=off -fno-omit-frame-pointer "
               f"-fsanitize=address,undefined -fno-sanitize-recover=undefined -shared-libasan -o {tmp} {src} -lm")
        if os.system(cmd) != 0:
            raise RuntimeError(f"failed: {cmd}")
        os.replace(tmp, out)
    return out


SAN_CC = "/opt/rocm/llvm/bin/clang"


@lru_cache(maxsize=1)
def _lib():
    # NPO_LIB selects another build of oracle.c (the sanitizer build of the host sanitizer tests)
    path = os.environ.get("NPO_LIB") or _LIB_PATH
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build_lib()
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.npo_active_set.argtypes = [vp, vp, i32, i32, vp]
    lib.npo_active_set.restype = i32
    lib.npo_delta_step.argtypes = [i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.npo_delta_step.restype = i32
    lib.npo_occupied_slots.argtypes = [i32, vp, vp]
    lib.npo_occupied_slots.restype = i32
    lib.npo_copy_bundles.argtypes = [vp, vp, i64, vp, vp, i32]
    lib.npo_copy_bundles.restype = None
    lib.npo_sparse_ffn.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    lib.npo_sparse_ffn.restype = i32
    lib.npo_sparse_ffn_act.argtypes = [vp, i32, i32, vp, i32, vp, i32, vp]
    lib.npo_sparse_ffn_act.restype = i32
    lib.npo_window_target.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp]
    lib.npo_window_target.restype = i32
    lib.npo_level_target.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp]
    lib.npo_level_target.restype = i32
    lib.npo_compact_step.argtypes = [i32, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.npo_compact_step.restype = i32
    lib.npo_move_bundles.argtypes = [vp, i64, vp, vp, i32]
    lib.npo_move_bundles.restype = None
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class CapacityError(RuntimeError):
    """|A_t| > K_max: the oracle refuses the step and leaves its state unchanged."""


def active_set(mask_g: np.ndarray, mask_u: np.ndarray | None, M: int, mode: int) -> np.ndarray:
    """Ascending neuron IDs of the active set built from one or two centroid masks."""
    g = _c(mask_g, np.uint64)
    u = _c(mask_u if mask_u is not None else mask_g, np.uint64)
    assert g.size * 64 >= M and u.size * 64 >= M
    out = np.empty(max(M, 1), dtype=np.int32)
    n = _lib().npo_active_set(g.ctypes.data, u.ctypes.data, M, mode, out.ctypes.data)
    if n < 0:
        raise ValueError(f"unknown mask mode {mode}")
    return out[:n].copy()


@dataclass
class StepResult:
    d_in: np.ndarray      # ascending incoming neuron IDs
    slot_in: np.ndarray   # slot (compact layout: position) assigned to each incoming neuron
    d_out: np.ndarray     # ascending outgoing neuron IDs
    mv_src: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))  # compact layout:
    mv_dst: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))  # rows moved src -> dst


_NEVER = -(1 << 30)


class OracleLayer:
    """Slot map, owner table and (optionally) the K_max-row buffer of one sparse layer.

    window = 1: the buffer holds exactly the active set (NeuroPrefetcher section 3.4).
    window = k > 1: it also keeps neurons active in the last k - 1 tokens, capacity
    permitting (LLM in a flash, section 3.1; see npo_window_target).
    levels (uint8 [M], values < n_levels): it keeps resident neurons by frequency level,
    capacity permitting (DynamicInfer, key design 2; see npo_level_target).
    layout "compact": the rows of the active set always fill positions 0 .. |S|-1 (LLM in a
    flash, section 3.3; see npo_compact_step); slot_map then maps a neuron to its position."""

    def __init__(self, M: int, K: int, R: int, d: int, keep_buffer: bool = True, window: int = 1,
                 levels: np.ndarray | None = None, n_levels: int = 0, layout: str = "slots"):
        assert window >= 1 and layout in ("slots", "compact")
        assert layout == "slots" or (window == 1 and levels is None)
        self.layout = layout
        self.n_occ = 0
        assert levels is None or (window == 1 and n_levels >= 1 and len(levels) == M)
        self.M, self.K, self.R, self.d, self.window = M, K, R, d, window
        self.levels = None if levels is None else _c(levels, np.uint8)
        self.n_levels = n_levels if levels is not None else 0
        self.slot_map = np.full(M, -1, dtype=np.int32)
        self.owner = np.full(K, -1, dtype=np.int32)
        self.last_t = np.full(M, _NEVER, dtype=np.int32)
        self.t = 0
        self.buf = np.zeros((K, R, d), dtype=np.uint16) if keep_buffer else None

    def reset(self) -> None:
        self.slot_map.fill(-1)
        self.owner.fill(-1)
        self.n_occ = 0
        self.last_t.fill(_NEVER)
        self.t = 0
        if self.buf is not None:
            self.buf.fill(0)

    def target(self, S: np.ndarray) -> np.ndarray:
        """The resident set this token moves to (S itself for window 1)."""
        S = _c(S, np.int32)
        if self.levels is not None:
            R = np.empty(self.M, dtype=np.int32)
            m = _lib().npo_level_target(self.M, self.K, self.n_levels, self.levels.ctypes.data,
                                        self.slot_map.ctypes.data, S.ctypes.data, S.size, R.ctypes.data)
            if m == -2:
                raise CapacityError(f"|S|={S.size} > K_max={self.K}")
            if m < 0:
                raise ValueError("invalid active set or levels")
            return R[:m].copy()
        if self.window == 1:
            if S.size > self.K:
                raise CapacityError(f"|S|={S.size} > K_max={self.K}")
            return S
        R = np.empty(self.M, dtype=np.int32)
        m = _lib().npo_window_target(self.M, self.K, self.window, self.t, self.last_t.ctypes.data,
                                     self.slot_map.ctypes.data, S.ctypes.data, S.size, R.ctypes.data)
        if m == -2:
            raise CapacityError(f"|S|={S.size} > K_max={self.K}")
        if m < 0:
            raise ValueError("invalid active set")
        return R[:m].copy()

    def active_slots(self, S: np.ndarray) -> np.ndarray:
        """Ascending slots of the active neurons (the rows the FFN reads)."""
        return np.sort(self.slot_map[_c(S, np.int32)])

    def step(self, S: np.ndarray) -> StepResult:
        S = _c(S, np.int32)
        if self.layout == "compact":
            return self._compact_step(S)
        res = self._move_to(self.target(S))
        self.last_t[S] = self.t
        self.t += 1
        return res

    def _move_to(self, S: np.ndarray) -> StepResult:
        S = _c(S, np.int32)
        d_in = np.empty(self.K, dtype=np.int32)
        slot_in = np.empty(self.K, dtype=np.int32)
        d_out = np.empty(self.K, dtype=np.int32)
        n_in = ctypes.c_int32(0)
        n_out = ctypes.c_int32(0)
        rc = _lib().npo_delta_step(self.M, self.K, self.slot_map.ctypes.data, self.owner.ctypes.data,
                                   S.ctypes.data, S.size, d_in.ctypes.data, slot_in.ctypes.data,
                                   ctypes.byref(n_in), d_out.ctypes.data, ctypes.byref(n_out))
        if rc == _ECAPACITY:
            raise CapacityError(f"|S|={S.size} > K_max={self.K}")
        if rc != _OK:
            raise ValueError("invalid active set")
        return StepResult(d_in[: n_in.value].copy(), slot_in[: n_in.value].copy(),
                          d_out[: n_out.value].copy())

    def _compact_step(self, S: np.ndarray) -> StepResult:
        K = self.K
        d_in, pos_in, d_out = (np.empty(K, dtype=np.int32) for _ in range(3))
        mv_src, mv_dst = np.empty(K, dtype=np.int32), np.empty(K, dtype=np.int32)
        n_occ, n_in, n_out, n_mv = (ctypes.c_int32(v) for v in (self.n_occ, 0, 0, 0))
        rc = _lib().npo_compact_step(self.M, K, self.slot_map.ctypes.data, self.owner.ctypes.data,
                                     ctypes.byref(n_occ), S.ctypes.data, S.size, d_in.ctypes.data,
                                     pos_in.ctypes.data, ctypes.byref(n_in), d_out.ctypes.data,
                                     ctypes.byref(n_out), mv_src.ctypes.data, mv_dst.ctypes.data,
                                     ctypes.byref(n_mv))
        if rc == _ECAPACITY:
            raise CapacityError(f"|S|={S.size} > K_max={K}")
        if rc != _OK:
            raise ValueError("invalid active set")
        self.n_occ = n_occ.value
        self.t += 1
        return StepResult(d_in[: n_in.value].copy(), pos_in[: n_in.value].copy(), d_out[: n_out.value].copy(),
                          mv_src[: n_mv.value].copy(), mv_dst[: n_mv.value].copy())

    def copy_bundles(self, store: np.ndarray, res: StepResult) -> None:
        """Moves of a compact step first (buf[mv_dst] = buf[mv_src]), then
        buf[slot_in[k]] = store[d_in[k]] (byte copy); store is uint16 [M][R][d]."""
        assert self.buf is not None
        if res.mv_src.size:
            _lib().npo_move_bundles(self.buf.ctypes.data, self.R * self.d, res.mv_src.ctypes.data,
                                    res.mv_dst.ctypes.data, res.mv_src.size)
        st = store.reshape(-1)
        assert st.dtype == np.uint16 and st.flags.c_contiguous and st.size >= self.M * self.R * self.d
        _lib().npo_copy_bundles(self.buf.ctypes.data, st.ctypes.data, self.R * self.d,
                                res.d_in.ctypes.data, res.slot_in.ctypes.data, res.d_in.size)

    def copy_given_bundles(self, bundles: np.ndarray, res: StepResult) -> None:
        """Same as copy_bundles, with bundles[k] already holding neuron d_in[k]'s bundle."""
        assert self.buf is not None
        if res.mv_src.size:
            _lib().npo_move_bundles(self.buf.ctypes.data, self.R * self.d, res.mv_src.ctypes.data,
                                    res.mv_dst.ctypes.data, res.mv_src.size)
        b = _c(bundles, np.uint16).reshape(-1)
        ids = np.arange(res.d_in.size, dtype=np.int32)
        _lib().npo_copy_bundles(self.buf.ctypes.data, b.ctypes.data, self.R * self.d,
                                ids.ctypes.data, res.slot_in.ctypes.data, res.d_in.size)

    def occupied_slots(self) -> np.ndarray:
        out = np.empty(self.K, dtype=np.int32)
        n = _lib().npo_occupied_slots(self.K, self.owner.ctypes.data, out.ctypes.data)
        return out[:n].copy()


def sparse_ffn(store: np.ndarray, R: int, d: int, ids: np.ndarray, x: np.ndarray, act: str = "relu") -> np.ndarray:
    """fp64 y[d] = sum over ids (in the order given) of down_i * h_i; store is uint16 [*][R][d].
    h_i = act(gate_i . x) * (up_i . x) (R = 3) or act(up_i . x) (R = 2), act "relu" or "silu"."""
    st = store.reshape(-1)
    assert st.dtype == np.uint16 and st.flags.c_contiguous
    ids = _c(ids, np.int32)
    if ids.size:
        assert ids.min() >= 0 and (int(ids.max()) + 1) * R * d <= st.size
    x = _c(x, np.float32)
    assert x.size == d
    y = np.empty(d, dtype=np.float64)
    rc = _lib().npo_sparse_ffn_act(st.ctypes.data, R, d, ids.ctypes.data, ids.size, x.ctypes.data,
                                   ACTS[act], y.ctypes.data)
    if rc != _OK:
        raise ValueError(f"unsupported bundle rows {R} or activation {act}")
    return y
