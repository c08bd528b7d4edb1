"""GPU parity of the retention by frequency level (DynamicInfer key design 2; the oracle's
npo_level_target): delta lists, slot map, owner table, the FFN's slot list and the buffer
bit-exact, y within max-abs 2e-2 / relative L2 5e-3, under capacity pressure, through
np_decode_step (direct launches and graph replay) and the per-layer calls."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, compare_state, make_layer, torch_mod
from workload.gen import Workload, small_config

pytestmark = pytest.mark.gpu

SHAPES = [
    small_config(930, L=2, d=512, M=600, K=150, C=6, mode="union", m=60, swap=10, T=12),
    small_config(931, L=2, d=4096, M=1500, K=500, C=5, mode="union", m=200, swap=30, T=10),
    small_config(932, L=1, d=1000, M=900, K=400, C=4, mode="intersect", m=380, swap=40, T=10, act="silu"),
]


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available()
    return t


def set_levels(layers, wl, n_levels):
    for l, layer in enumerate(layers):
        layer.set_levels(wl.frequency_levels(l, n_levels), n_levels)


@pytest.mark.parametrize("n_levels", [1, 4, 16])
@pytest.mark.parametrize("path", ["direct", "graph", "calls"])
@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: f"d{c.d}_M{c.M}_K{c.K}_{c.mode}")
def test_levels_parity(torch, cfg, path, n_levels):
    from delta_prefetched_ffn_amd import binding as B
    print(f"[levels] {cfg.num} {path} n_levels={n_levels}", flush=True)
    B.decode_use_graphs(path == "graph")
    wl = Workload(cfg)
    layers, stores = zip(*[make_layer(wl, l) for l in range(cfg.L)])
    set_levels(layers, wl, n_levels)
    orc = OracleRun(wl, n_levels=n_levels)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    cs = torch.cuda.Stream()
    loads = 0
    for t in range(cfg.T):
        if path == "calls":
            for l, layer in enumerate(layers):
                g, u = (int(v) for v in wl.cids()[t, l])
                layer.delta_assign(g, u, cs.cuda_stream)
                layer.sparse_ffn(x[t, l].data_ptr(), y[t, l].data_ptr(), cs.cuda_stream)  # read-through
        else:
            B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), cs.cuda_stream, cs.cuda_stream)
        for l, layer in enumerate(layers):
            st = layer.read_state()
            S, res = orc.step(t, l, stores[l])
            compare_state(st, orc.layers[l], res, S, f"levels={n_levels} t={t} l={l}")
            assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"levels={n_levels} t={t} l={l}: buffer"
            assert layer.info()["n_in"] == res.d_in.size
            loads += res.d_in.size
    torch.cuda.synchronize()
    assert sum(layer.counters()[1] for layer in layers) == loads
    yh = y.cpu().numpy()
    for t in range(cfg.T):
        for l in range(cfg.L):
            S = orc.active(t, l)
            check_y(yh[t, l], O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act), f"t={t} l={l}")
    for layer in layers:
        layer.close()
    B.decode_use_graphs(False)


def test_levels_reduce_loads_and_zero_is_the_exact_rule(torch):
    from delta_prefetched_ffn_amd import binding as B
    cfg = SHAPES[0]
    wl = Workload(cfg)
    x = torch.from_numpy(wl.x_all()).cuda()
    totals, outs = {}, {}
    for n_levels in (None, 0, 4):
        layers = [make_layer(wl, l)[0] for l in range(cfg.L)]
        for layer in layers:
            layer.set_ffn_reduce("ordered")  # for the bitwise comparison below
        if n_levels is not None:
            set_levels(layers, wl, n_levels) if n_levels else [layer.set_levels(None, 0) for layer in layers]
        y = torch.zeros_like(x)
        for t in range(cfg.T):
            B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), 0, 0)
        torch.cuda.synchronize()
        totals[n_levels] = sum(layer.counters()[1] for layer in layers)
        outs[n_levels] = y.cpu().numpy()
        for layer in layers:
            layer.close()
    assert totals[None] == totals[0] and totals[4] < totals[0]
    assert np.array_equal(outs[None].view(np.uint32), outs[0].view(np.uint32))


def test_set_levels_checks(torch):
    from delta_prefetched_ffn_amd import binding as B
    wl = Workload(SHAPES[0])
    c = wl.cfg
    layer = make_layer(wl, 0)[0]
    lv = wl.frequency_levels(0, 4)
    for n in (-1, 17):
        with pytest.raises(B.NPError) as e:
            layer.set_levels(np.zeros(c.M), n)
        assert e.value.status == B.NP_EINVAL
    bad = lv.copy()
    bad[5] = 4                                   # not below n_levels
    with pytest.raises(B.NPError) as e:
        layer.set_levels(bad, 4)
    assert e.value.status == B.NP_EINVAL
    layer.set_window(3)
    with pytest.raises(B.NPError) as e:
        layer.set_levels(lv, 4)                  # a window excludes levels
    assert e.value.status == B.NP_EINVAL
    layer.set_window(1)
    layer.set_levels(lv, 4)
    with pytest.raises(B.NPError) as e:
        layer.set_window(2)                      # and levels exclude a window
    assert e.value.status == B.NP_EINVAL
    g, u = (int(v) for v in wl.cids()[0, 0])
    layer.delta_assign(g, u, 0)
    with pytest.raises(B.NPError) as e:
        layer.set_levels(lv, 2)                  # not before the first assignment
    assert e.value.status == B.NP_ESTATE
    layer.scatter_rows(0)
    torch.cuda.synchronize()
    layer.reset()
    layer.set_levels(None, 0)                    # fine again after a reset
    layer.close()
