"""Seeded synthetic inputs for the delta-prefetched sparse FFN.

This module produces inputs only: centroid mask tables, per-token centroid
IDs, bf16 weight bundles and fp32 activation vectors. It holds none of the
method's arithmetic (no mask combination, no set difference, no slot
assignment, no dot products); the CPU oracle and the HIP path both consume
what it produces.

The five workloads stand in for the model shapes and decode runs of the
NeuroPrefetcher paper (page "NeuroPrefetcher: Storage-Aware Sparse LLM
Inference via Delta Prefetching", sections 3.4 and 4.5: gate/up centroid
masks per sparse layer, 82-85% token-to-token reuse of active rows) and of
LLM in a flash (section 3.2: the [up|down] bundle of a non-gated ReLU FFN).
No dataset or trained model is used.

Randomness:
  * mask tables, centroid IDs and trajectories: NumPy PCG64 seeded with
    SeedSequence([root_seed, config, layer, purpose]);
  * weights and activations: the counter-based SplitMix64 + Box-Muller
    generator in wlgen.c, keyed by the same SeedSequence, so any bundle can
    be regenerated on its own.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

ROOT_SEED = 20261202

# SeedSequence purposes
P_BASE, P_GATE, P_UP, P_WEIGHTS, P_X, P_CIDS, P_TRAJ, P_PTOKEN = 0, 1, 2, 3, 4, 5, 6, 7

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwlgen.so")


def build_lib(force: bool = False) -> str:
    """Compile wlgen.c into libwlgen.so next to it (gcc, -O2, no fast-math)."""
    src = os.path.join(_HERE, "wlgen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = f"gcc -O2 -std=c11 -fPIC -shared -pthread -o {tmp} {src} -lm"
        if os.system(cmd) != 0:
            raise RuntimeError(f"failed: {cmd}")
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


@lru_cache(maxsize=1)
def _lib():
    if not os.path.exists(_LIB_PATH):
        build_lib()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
    vp = ctypes.c_void_p
    lib.wl_fill_bf16.argtypes = [vp, u64, u64, u64, f64, ctypes.c_int]
    lib.wl_fill_f32.argtypes = [vp, u64, u64, u64, f64, ctypes.c_int]
    lib.wl_fill_bundles_bf16.argtypes = [vp, u64, vp, i64, u64, f64]
    for f in (lib.wl_fill_bf16, lib.wl_fill_f32, lib.wl_fill_bundles_bf16):
        f.restype = ctypes.c_int
    return lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def stream_key(*words: int) -> int:
    """64-bit key of a counter-based stream, from SeedSequence(words)."""
    return int(np.random.SeedSequence(list(words)).generate_state(1, dtype=np.uint64)[0])


def rng_for(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words))))


def fill_normal_bf16(count: int, key: int, first: int = 0, std: float = 0.02,
                     out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of std * N(0,1), values [first, first+count) of stream key."""
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == count
    _lib().wl_fill_bf16(out.ctypes.data, key, first, count, std, _threads())
    return out


def fill_normal_f32(count: int, key: int, first: int = 0, std: float = 1.0,
                    out: np.ndarray | None = None) -> np.ndarray:
    if out is None:
        out = np.empty(count, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == count
    _lib().wl_fill_f32(out.ctypes.data, key, first, count, std, _threads())
    return out


def bits_to_words(bits: np.ndarray, n_bits: int) -> np.ndarray:
    """Pack a bool vector into uint64 words: bit b of word w is element 64*w + b."""
    W = (n_bits + 63) // 64
    padded = np.zeros(W * 64, dtype=np.uint8)
    padded[:n_bits] = bits[:n_bits].astype(np.uint8)
    return np.packbits(padded, bitorder="little").view("<u8").astype(np.uint64)


def ids_to_words(ids, n_bits: int) -> np.ndarray:
    bits = np.zeros(n_bits, dtype=bool)
    bits[np.asarray(ids, dtype=np.int64)] = True
    return bits_to_words(bits, n_bits)


@dataclass(frozen=True)
class Config:
    """One synthetic workload: shapes, centroid recipe, steps."""
    num: int              # config number (enters every seed)
    name: str
    L: int                # sparse layers
    d: int                # d_model
    M: int                # d_ff (neurons)
    R: int                # rows per bundle: 3 = [gate|up|down^T], 2 = [up|down^T]
    K: int                # K_max slots per layer
    C: int                # centroids per projection table
    mode: str             # "union" | "intersect" | "single"
    T: int                # decode steps
    recipe: str = "swap"  # "swap" (base set with swapped members) | "trajectory"
    m: int = 0            # swap recipe: mask size
    swap: int = 0         # swap recipe: members replaced by non-members
    active: int = 0       # trajectory recipe: |A_t|
    p_lo: float = 0.0     # trajectory recipe: persistence range
    p_hi: float = 0.0
    w_std: float = 0.02
    act: str = "relu"     # activation of the model's FFN: "relu" | "silu" (SwiGLU gate)

    @property
    def W(self) -> int:
        return (self.M + 63) // 64

    @property
    def n_proj(self) -> int:
        return 1 if self.mode == "single" else 2

    @property
    def bundle_elems(self) -> int:
        return self.R * self.d

    @property
    def bundle_bytes(self) -> int:
        return 2 * self.R * self.d


CONFIGS = {
    1: Config(1, "tiny d256 M1024 gated ReLU", L=1, d=256, M=1024, R=3, K=384, C=64,
              mode="union", T=16, m=192, swap=31),
    2: Config(2, "Llama-2-7B-shaped sparse FFN", L=31, d=4096, M=11008, R=3, K=4096, C=256,
              mode="union", T=256, m=1130, swap=102),
    3: Config(3, "Llama-2-13B-shaped sparse FFN", L=39, d=5120, M=13824, R=3, K=5120, C=512,
              mode="union", T=256, m=1420, swap=128),
    4: Config(4, "OPT-6.7B-shaped non-gated ReLU FFN", L=31, d=4096, M=16384, R=2, K=3072, C=256,
              mode="single", T=256, m=1065, swap=88),
    5: Config(5, "large d7168 M28672 low-overlap", L=47, d=7168, M=28672, R=3, K=6144, C=128,
              mode="union", T=128, recipe="trajectory", active=2867, p_lo=0.70, p_hi=0.90),
    # The low-overlap stress case of DynamicInfer (adjacent-token Jaccard distance 0.70-0.75,
    # i.e. about 45% persistence) at the Llama-2-7B shape.
    9: Config(9, "Llama-2-7B-shaped low-overlap stress", L=31, d=4096, M=11008, R=3, K=4096, C=128,
              mode="union", T=128, recipe="trajectory", active=1324, p_lo=0.40, p_hi=0.50),
    # The paper's own model shape (Mistral-7B: d 4096, d_ff 14336, SwiGLU), its active set the
    # intersection of the gate and up masks, at its three K_max budgets (62 / 50 / 31%
    # sparsity). Each mask keeps K_max - s members of a base set of K_max neurons; the
    # intersection then has about K_max (1 - s/K_max)^2 neurons and consecutive tokens share
    # about (1 - s/K_max)^2 of them (0.84 at s/K_max = 0.0835).
    6: Config(6, "Mistral-7B-shaped SwiGLU FFN, K_max 5500", L=31, d=4096, M=14336, R=3, K=5500,
              C=512, mode="intersect", T=256, m=5500, swap=459, act="silu"),
    7: Config(7, "Mistral-7B-shaped SwiGLU FFN, K_max 7168", L=31, d=4096, M=14336, R=3, K=7168,
              C=512, mode="intersect", T=256, m=7168, swap=599, act="silu"),
    8: Config(8, "Mistral-7B-shaped SwiGLU FFN, K_max 9865", L=31, d=4096, M=14336, R=3, K=9865,
              C=512, mode="intersect", T=256, m=9865, swap=824, act="silu"),
}


def small_config(num: int, *, L=2, d=64, M=200, R=3, K=96, C=8, mode="union", T=6, m=40,
                 swap=6, name="test shape", act="relu") -> Config:
    """A reduced shape for fast tests (same recipe, own seeds via `num`)."""
    return Config(num, name, L=L, d=d, M=M, R=R, K=K, C=C, mode=mode, T=T, m=m, swap=swap, act=act)


class Workload:
    """Lazily generated inputs of one Config."""

    def __init__(self, cfg: Config, seed: int = ROOT_SEED):
        self.cfg = cfg
        self.seed = seed
        self._masks: dict[int, np.ndarray] = {}
        self._cids: np.ndarray | None = None

    # ---------------------------------------------------------------- masks
    def _swap_table(self, l: int, purpose: int, base: np.ndarray) -> np.ndarray:
        c = self.cfg
        rng = rng_for(self.seed, c.num, l, purpose)
        in_base = np.zeros(c.M, dtype=bool)
        in_base[base] = True
        others = np.nonzero(~in_base)[0]
        table = np.empty((c.C, c.W), dtype=np.uint64)
        for k in range(c.C):
            keep = rng.choice(base, size=c.m - c.swap, replace=False)
            add = rng.choice(others, size=c.swap, replace=False)
            table[k] = ids_to_words(np.concatenate([keep, add]), c.M)
        return table

    def _trajectory_tables(self, l: int) -> np.ndarray:
        """Config-5 style: A_t built with per-token persistence, split into gate/up masks.

        A_0 is `active` uniform neurons. For t >= 1, round(p_t * |A_{t-1}|) uniform members
        of A_{t-1} are kept and the rest is drawn uniformly from the complement; p_t is drawn
        per token from U[p_lo, p_hi] and shared by all layers. Each member of A_t goes to
        gate-only / up-only / both with probability 0.2 / 0.2 / 0.6, so the union of the two
        masks is A_t. Step t uses table entry pi(t) for a seeded permutation pi.
        """
        c = self.cfg
        assert c.C >= c.T
        rng = rng_for(self.seed, c.num, l, P_TRAJ)
        p = self.token_persistence()
        perm = self.trajectory_perm()
        gate = np.zeros((c.C, c.W), dtype=np.uint64)
        up = np.zeros((c.C, c.W), dtype=np.uint64)
        cur = np.sort(rng.choice(c.M, size=c.active, replace=False))
        for t in range(c.T):
            if t > 0:
                keep_n = int(round(p[t] * cur.size))
                keep = rng.choice(cur, size=keep_n, replace=False)
                mark = np.zeros(c.M, dtype=bool)
                mark[cur] = True
                comp = np.nonzero(~mark)[0]
                add = rng.choice(comp, size=c.active - keep_n, replace=False)
                cur = np.sort(np.concatenate([keep, add]))
            u = rng.random(cur.size)
            g_ids = cur[(u < 0.2) | (u >= 0.4)]
            u_ids = cur[u >= 0.2]
            gate[perm[t]] = ids_to_words(g_ids, c.M)
            up[perm[t]] = ids_to_words(u_ids, c.M)
        return np.stack([gate, up])

    def token_persistence(self) -> np.ndarray:
        c = self.cfg
        rng = rng_for(self.seed, c.num, 0, P_PTOKEN)
        return rng.uniform(c.p_lo, c.p_hi, size=c.T)

    def trajectory_perm(self) -> np.ndarray:
        c = self.cfg
        return rng_for(self.seed, c.num, 0, P_CIDS).permutation(c.C)

    def masks(self, l: int) -> np.ndarray:
        """uint64 [n_proj][C][W] centroid mask tables of layer l (gate, up) or (single)."""
        if l not in self._masks:
            c = self.cfg
            if c.recipe == "trajectory":
                self._masks[l] = self._trajectory_tables(l)
            else:
                rng = rng_for(self.seed, c.num, l, P_BASE)
                base = rng.choice(c.M, size=c.m, replace=False)
                tabs = [self._swap_table(l, P_GATE, base)]
                if c.n_proj == 2:
                    tabs.append(self._swap_table(l, P_UP, base))
                self._masks[l] = np.stack(tabs)
        return self._masks[l]

    def frequency_levels(self, l: int, n_levels: int) -> np.ndarray:
        """uint8 [M]: each neuron's activation frequency over layer l's centroid masks (the
        fraction of the gate and up masks that hold it), quantised to n_levels equal-width
        levels (0 = rarest). A stand-in for offline activation statistics."""
        c = self.cfg
        tabs = self.masks(l)
        bits = np.unpackbits(tabs.view(np.uint8).reshape(tabs.shape[0], c.C, -1), axis=-1,
                             bitorder="little")[:, :, : c.M]
        f = bits.reshape(-1, c.M).mean(axis=0)
        return np.minimum((f * n_levels).astype(np.int64), n_levels - 1).astype(np.uint8)

    # ----------------------------------------------------------------- cids
    def cids(self) -> np.ndarray:
        """int32 [T][L][2]: (gate cid, up cid) per step and layer; single mode repeats it.

        Swap recipe: uniform, independent per (step, layer, projection). The construction
        bounds |mask_g| + |mask_u| <= 2m, and every built-in config keeps 2m <= K_max, so no
        draw can exceed the slot capacity (for single mode m <= K_max).
        """
        if self._cids is None:
            c = self.cfg
            if c.recipe == "trajectory":
                perm = self.trajectory_perm()
                cid = np.repeat(perm[: c.T, None], c.L, axis=1)
                self._cids = np.stack([cid, cid], axis=-1).astype(np.int32)
            else:
                rng = rng_for(self.seed, c.num, 0, P_CIDS)
                g = rng.integers(0, c.C, size=(c.T, c.L))
                u = rng.integers(0, c.C, size=(c.T, c.L)) if c.n_proj == 2 else g
                self._cids = np.stack([g, u], axis=-1).astype(np.int32)
        return self._cids

    # --------------------------------------------------------------- values
    def weight_key(self, l: int) -> int:
        return stream_key(self.seed, self.cfg.num, l, P_WEIGHTS)

    def store(self, l: int, out: np.ndarray | None = None) -> np.ndarray:
        """bf16 bits uint16 [M][R][d]: row store of layer l (bundle n = rows of neuron n)."""
        c = self.cfg
        n = c.M * c.R * c.d
        if out is not None:
            out = out.reshape(-1)
        arr = fill_normal_bf16(n, self.weight_key(l), 0, c.w_std, out)
        return arr.reshape(c.M, c.R, c.d)

    def bundles(self, l: int, ids) -> np.ndarray:
        """bf16 bits uint16 [len(ids)][R][d]: bundles of the given neurons, regenerated."""
        c = self.cfg
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        out = np.empty((ids.size, c.R, c.d), dtype=np.uint16)
        if ids.size:
            _lib().wl_fill_bundles_bf16(out.ctypes.data, self.weight_key(l), ids.ctypes.data,
                                        ids.size, c.bundle_elems, c.w_std)
        return out

    def x(self, t: int, l: int) -> np.ndarray:
        c = self.cfg
        return fill_normal_f32(c.d, stream_key(self.seed, c.num, l, P_X), t * c.d, 1.0)

    def x_all(self) -> np.ndarray:
        """fp32 [T][L][d]."""
        c = self.cfg
        out = np.empty((c.L, c.T * c.d), dtype=np.float32)
        for l in range(c.L):
            fill_normal_f32(c.T * c.d, stream_key(self.seed, c.num, l, P_X), 0, 1.0, out[l])
        return np.ascontiguousarray(out.reshape(c.L, c.T, c.d).transpose(1, 0, 2))
