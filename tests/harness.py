"""Shared helpers for the GPU parity tests: build layers from a Workload, run the
HIP path through the C ABI, and run the CPU oracle beside it.

Tolerance for y (fp32 accumulation of bf16 x fp32 products against the fp64
oracle): max |dy| <= 2e-2 and ||dy||_2 / ||y||_2 <= 5e-3 per (step, layer).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O
from workload.gen import Workload

MAX_ABS = 2e-2
REL_L2 = 5e-3


def torch_mod():
    import torch
    return torch


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "") -> None:
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    diff = y_gpu - y_ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(y_ref))
    rel = float(np.linalg.norm(diff)) / nrm if nrm > 0 else float(np.linalg.norm(diff))
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


def upload_store(store_u16: np.ndarray, where: str):
    """Place a uint16 [M][R][d] store in HBM ('device') or pinned host memory ('host')."""
    torch = torch_mod()
    t = torch.from_numpy(store_u16.reshape(-1).view(np.int16))
    if where == "device":
        return t.to("cuda")
    p = torch.empty(t.numel(), dtype=torch.int16, pin_memory=True)
    p.copy_(t)
    return p


def make_layer(wl: Workload, l: int, where: str = "device", store: np.ndarray | None = None):
    from delta_prefetched_ffn_amd import binding as B
    c = wl.cfg
    if store is None:
        store = wl.store(l)
    dev_store = upload_store(store, where)
    layer = B.Layer(d_model=c.d, d_ff=c.M, k_max=c.K, n_rows=c.R, masks=wl.masks(l),
                    mask_mode=B.MODES[c.mode], act=B.ACTS[c.act], row_store=dev_store.data_ptr(), keepalive=dev_store)
    return layer, store


class OracleRun:
    """The oracle's state for every layer of a workload."""

    def __init__(self, wl: Workload, keep_buffer: bool = True, window: int = 1, n_levels: int = 0,
                 layout: str = "slots"):
        c = wl.cfg
        self.wl = wl
        self.layers = [O.OracleLayer(c.M, c.K, c.R, c.d, keep_buffer=keep_buffer, window=window,
                                     levels=wl.frequency_levels(l, n_levels) if n_levels else None,
                                     n_levels=n_levels, layout=layout)
                       for l in range(c.L)]
        self.mode = O.MODES[c.mode]

    def active(self, t: int, l: int) -> np.ndarray:
        tabs = self.wl.masks(l)
        cid = self.wl.cids()[t, l]
        return O.active_set(tabs[0][cid[0]], tabs[-1][cid[1]], self.wl.cfg.M, self.mode)

    def step(self, t: int, l: int, store: np.ndarray | None = None):
        S = self.active(t, l)
        res = self.layers[l].step(S)
        if store is not None and self.layers[l].buf is not None:
            self.layers[l].copy_bundles(store, res)
        return S, res


def compare_state(st: dict, ol: O.OracleLayer, res: O.StepResult, S: np.ndarray, what: str) -> None:
    assert st["err"] == 0, f"{what}: device error bits {st['err']}"
    assert np.array_equal(st["d_in"], res.d_in), f"{what}: d_in differs"
    assert np.array_equal(st["slot_in"], res.slot_in), f"{what}: slot_in differs"
    assert np.array_equal(st["d_out"], res.d_out), f"{what}: d_out differs"
    assert np.array_equal(st["slot_map"], ol.slot_map), f"{what}: slot_map differs"
    assert np.array_equal(st["owner"], ol.owner), f"{what}: owner differs"
    assert np.array_equal(st["act"], ol.active_slots(S)), f"{what}: active slot list differs"
    if ol.window == 1 and ol.levels is None:
        assert np.array_equal(st["act"], ol.occupied_slots()), f"{what}: occupied slots differ"
    assert st["act"].size == S.size
