"""Different layers driven from different host threads at the same time (the C ABI allows it:
a layer is not thread-safe, but separate layers are): two threads each run their own workload's
decode steps on their own streams, one with its row stores in HBM (one queue), two with pinned
host stores (token launches, so two of them can run on the GPU at once); afterwards each
workload's state, whole buffer and y match the oracle exactly as in a single-threaded run. ctypes releases the GIL around every
library call, so the two threads' host work and enqueues really interleave."""
import threading

import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, make_layer, torch_mod
from workload.gen import Workload, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available()
    return t


def test_three_threads_three_workloads(torch):
    from delta_prefetched_ffn_amd import binding as B
    B.decode_use_graphs(False)
    runs = []
    for k, (where, cfg) in enumerate([
            ("device", small_config(1500, L=3, d=512, M=900, K=300, C=5, mode="union", m=120, swap=20, T=24)),
            ("host", small_config(1501, L=2, d=1000, M=700, K=260, C=4, mode="intersect", m=200, swap=30, T=24,
                                  act="silu")),
            ("host", small_config(1502, L=4, d=256, M=600, K=200, C=5, mode="union", m=80, swap=15, T=24))]):
        wl = Workload(cfg)
        layers, stores = zip(*[make_layer(wl, l, where) for l in range(cfg.L)])
        x = torch.from_numpy(wl.x_all()).cuda()
        y = torch.zeros_like(x)
        cs = torch.cuda.Stream()
        ps = torch.cuda.Stream() if where == "host" else cs
        runs.append(dict(wl=wl, cfg=cfg, layers=layers, stores=stores, x=x, y=y, cs=cs, ps=ps, err=None))
    torch.cuda.synchronize()
    barrier = threading.Barrier(len(runs))

    def drive(r):
        try:
            barrier.wait()
            for t in range(r["cfg"].T):
                B.decode_step(r["layers"], r["wl"].cids()[t], r["x"][t].data_ptr(), r["y"][t].data_ptr(),
                              r["cs"].cuda_stream, r["ps"].cuda_stream)
            r["cs"].synchronize()
        except Exception as e:  # reported after the join
            r["err"] = e

    threads = [threading.Thread(target=drive, args=(r,)) for r in runs]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert all(not th.is_alive() for th in threads)
    for r in runs:
        assert r["err"] is None, r["err"]
    torch.cuda.synchronize()
    for r in runs:
        cfg, wl = r["cfg"], r["wl"]
        orc = OracleRun(wl)
        for t in range(cfg.T):
            for l in range(cfg.L):
                orc.step(t, l, r["stores"][l])
        for l, layer in enumerate(r["layers"]):
            st = layer.read_state()
            assert st["err"] == 0
            assert np.array_equal(st["slot_map"], orc.layers[l].slot_map)
            assert np.array_equal(st["owner"], orc.layers[l].owner)
            S = orc.active(cfg.T - 1, l)
            assert np.array_equal(st["act"], orc.layers[l].active_slots(S))
            assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"layer {l}: buffer"
        yh = r["y"].cpu().numpy()
        x_all = wl.x_all()
        for t in range(cfg.T):
            for l in range(cfg.L):
                S = orc.active(t, l)
                check_y(yh[t, l], O.sparse_ffn(r["stores"][l], cfg.R, cfg.d, S, x_all[t, l], cfg.act),
                        f"cfg {cfg.num} t={t} l={l}")
        for layer in r["layers"]:
            layer.close()
