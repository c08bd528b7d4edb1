"""GPU parity of the compacted buffer layout (LLM in a flash section 3.3; the oracle's
npo_compact_step): delta lists, position map, owner table, the moves, the FFN's row list and
the whole buffer (moved and stale rows included) bit-exact, y within max-abs 2e-2 / relative
L2 5e-3, through np_decode_step (direct launches, graph replay, one and two streams, device
and pinned-host row stores) and the per-layer calls."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, compare_state, make_layer, torch_mod
from workload.gen import Workload, small_config

pytestmark = pytest.mark.gpu

SHAPES = [
    small_config(940, L=2, d=512, M=600, K=150, C=6, mode="union", m=60, swap=10, T=12),
    small_config(941, L=2, d=4096, M=1500, K=500, C=5, mode="union", m=200, swap=30, T=10),
    small_config(942, L=1, d=1000, M=900, K=400, C=4, mode="intersect", m=380, swap=40, T=10, act="silu"),
    small_config(943, L=2, d=512, M=300, K=120, C=4, mode="single", R=2, m=100, swap=10, T=8),
]


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available()
    return t


@pytest.mark.parametrize("path", ["direct", "graph", "calls", "host2"])
@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: f"d{c.d}_M{c.M}_K{c.K}_{c.mode}_R{c.R}")
def test_compact_parity(torch, cfg, path):
    from delta_prefetched_ffn_amd import binding as B
    print(f"[compact] {cfg.num} {path}", flush=True)
    B.decode_use_graphs(path == "graph")
    wl = Workload(cfg)
    where = "host" if path == "host2" else "device"
    layers, stores = zip(*[make_layer(wl, l, where) for l in range(cfg.L)])
    for layer in layers:
        layer.set_layout("compact")
    orc = OracleRun(wl, layout="compact")
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    cs = torch.cuda.Stream()
    ps = torch.cuda.Stream() if path == "host2" else cs
    moves = 0
    for t in range(cfg.T):
        if path == "calls":
            for l, layer in enumerate(layers):
                g, u = (int(v) for v in wl.cids()[t, l])
                layer.delta_assign(g, u, cs.cuda_stream)
                layer.sparse_ffn(x[t, l].data_ptr(), y[t, l].data_ptr(), cs.cuda_stream)  # read-through
        else:
            B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), cs.cuda_stream, ps.cuda_stream)
        for l, layer in enumerate(layers):
            st = layer.read_state()
            S, res = orc.step(t, l, stores[l])
            what = f"{path} t={t} l={l}"
            compare_state(st, orc.layers[l], res, S, what)
            assert np.array_equal(st["act"], np.arange(S.size)), f"{what}: rows are not the prefix"
            src, dst = layer.read_moves()
            assert np.array_equal(src, res.mv_src) and np.array_equal(dst, res.mv_dst), f"{what}: moves"
            assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"{what}: buffer"
            moves += src.size
    torch.cuda.synchronize()
    assert moves > 0
    yh = y.cpu().numpy()
    for t in range(cfg.T):
        for l in range(cfg.L):
            S = orc.active(t, l)
            check_y(yh[t, l], O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act), f"t={t} l={l}")
    for layer in layers:
        layer.close()
    B.decode_use_graphs(False)


def test_set_layout_checks(torch):
    from delta_prefetched_ffn_amd import binding as B
    wl = Workload(SHAPES[0])
    layer = make_layer(wl, 0)[0]
    with pytest.raises(B.NPError) as e:
        B._check(B.lib().np_layer_set_layout(layer.h, 7))
    assert e.value.status == B.NP_EINVAL
    layer.set_window(2)
    with pytest.raises(B.NPError) as e:
        layer.set_layout("compact")              # the compact buffer holds exactly S
    assert e.value.status == B.NP_EINVAL
    layer.set_window(1)
    layer.set_layout("compact")
    with pytest.raises(B.NPError) as e:
        layer.set_window(3)
    assert e.value.status == B.NP_EINVAL
    with pytest.raises(B.NPError) as e:
        layer.set_levels(wl.frequency_levels(0, 2), 2)
    assert e.value.status == B.NP_EINVAL
    g, u = (int(v) for v in wl.cids()[0, 0])
    layer.delta_assign(g, u, 0)
    with pytest.raises(B.NPError) as e:
        layer.set_layout("slots")                # not before the first assignment
    assert e.value.status == B.NP_ESTATE
    layer.scatter_rows(0)
    torch.cuda.synchronize()
    layer.reset()
    layer.set_layout("slots")                    # fine again after a reset
    src, dst = layer.read_moves()
    assert src.size == 0 and dst.size == 0
    layer.close()
