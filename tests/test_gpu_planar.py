"""GPU parity of the planar slot buffers (one buffer per projection row, as NeuroPrefetcher
section 3.5 keeps the resident rows): the scatter kernels and the FFN's read-through split each
bundle into its planes; the slots, the buffer contents seen as bundles and y must be exactly
those of the interleaved arrangement (the oracle's), through every path."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, compare_state, make_layer, torch_mod
from workload.gen import Workload, small_config

pytestmark = pytest.mark.gpu

SHAPES = [
    small_config(980, L=2, d=512, M=600, K=150, C=6, mode="union", m=60, swap=10, T=8),
    small_config(981, L=2, d=4096, M=1500, K=500, C=5, mode="union", m=200, swap=30, T=6),
    small_config(982, L=2, d=1000, M=300, K=120, C=4, mode="single", R=2, m=100, swap=10, T=6, act="silu"),
]


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available()
    yield t
    from delta_prefetched_ffn_amd import binding as B
    B.decode_set_staging(0)
    B.decode_use_graphs(False)


@pytest.mark.parametrize("layout", ["slots", "compact"])
@pytest.mark.parametrize("path", ["direct", "graph", "calls", "host2", "staged"])
@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: f"d{c.d}_M{c.M}_K{c.K}_{c.mode}_R{c.R}")
def test_planar_parity(torch, cfg, path, layout):
    from delta_prefetched_ffn_amd import binding as B
    print(f"[planar] {cfg.num} {path} {layout}", flush=True)
    B.decode_use_graphs(path == "graph")
    B.decode_set_staging(5 * cfg.bundle_bytes if path == "staged" else 0)
    wl = Workload(cfg)
    where = "host" if path in ("host2", "staged") else "device"
    layers, stores = zip(*[make_layer(wl, l, where) for l in range(cfg.L)])
    for layer in layers:
        layer.set_planar(True)
        layer.set_layout(layout)
    orc = OracleRun(wl, layout=layout)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    cs = torch.cuda.Stream()
    ps = torch.cuda.Stream() if where == "host" else cs
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
            assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"{what}: buffer"
            sl = np.array([0, cfg.K - 1, cfg.K // 2], dtype=np.int32)
            assert np.array_equal(layer.read_rows(sl), orc.layers[l].buf[sl]), f"{what}: rows"
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for t in range(cfg.T):
        for l in range(cfg.L):
            S = orc.active(t, l)
            check_y(yh[t, l], O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act), f"t={t} l={l}")
    for layer in layers:
        layer.close()
    B.decode_use_graphs(False)
    B.decode_set_staging(0)


def test_planar_and_interleaved_agree_bitwise(torch):
    """Same inputs, ordered reduce: identical y and identical bundles."""
    from delta_prefetched_ffn_amd import binding as B
    cfg = SHAPES[1]
    wl = Workload(cfg)
    x = torch.from_numpy(wl.x_all()).cuda()
    outs, bufs = [], []
    for planar in (False, True):
        layers = [make_layer(wl, l)[0] for l in range(cfg.L)]
        for layer in layers:
            layer.set_planar(planar)
            layer.set_ffn_reduce("ordered")
        y = torch.zeros_like(x)
        for t in range(cfg.T):
            B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), 0, 0)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
        bufs.append([layer.read_rows() for layer in layers])
        for layer in layers:
            layer.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    for a, b in zip(*bufs):
        assert np.array_equal(a, b)


def test_set_planar_checks(torch):
    from delta_prefetched_ffn_amd import binding as B
    wl = Workload(SHAPES[0])
    layer = make_layer(wl, 0)[0]
    with pytest.raises(B.NPError) as e:
        B._check(B.lib().np_layer_set_planar(layer.h, 2))
    assert e.value.status == B.NP_EINVAL
    g, u = (int(v) for v in wl.cids()[0, 0])
    layer.delta_assign(g, u, 0)
    with pytest.raises(B.NPError) as e:
        layer.set_planar(True)
    assert e.value.status == B.NP_ESTATE
    layer.scatter_rows(0)
    torch.cuda.synchronize()
    layer.reset()
    layer.set_planar(True)
    layer.close()
