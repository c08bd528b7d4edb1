"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: delta lists, slot assignments, slot map, owner table, active-slot
list and buffer bytes. FFN output: max |dy| <= 2e-2 and relative L2 <= 5e-3
against the fp64 oracle; bit-exact on exact dyadic inputs.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, compare_state, make_layer, torch_mod, upload_store
from workload.gen import CONFIGS, Config, Workload, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available(), "GPU tests need a visible GPU"
    from delta_prefetched_ffn_amd import binding
    binding.lib()  # fails loudly if the HIP library is missing
    return t


def _stream(torch):
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("where", ["device", "host"])
def test_config1_single_layer_calls(torch, where):
    wl = Workload(CONFIGS[1])
    c = wl.cfg
    layer, store = make_layer(wl, 0, where)
    orc = OracleRun(wl)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    s = _stream(torch)
    for t in range(c.T):
        g, u = (int(v) for v in wl.cids()[t, 0])
        layer.delta_assign(g, u, s)
        layer.scatter_rows(s)
        layer.sparse_ffn(x[t, 0].data_ptr(), y[t, 0].data_ptr(), s)
        st = layer.read_state()
        S, res = orc.step(t, 0, store)
        compare_state(st, orc.layers[0], res, S, f"t={t}")
        assert np.array_equal(layer.read_rows(), orc.layers[0].buf), f"t={t}: buffer differs"
        check_y(y[t, 0].cpu().numpy(), O.sparse_ffn(store, c.R, c.d, S, x_all[t, 0], c.act), f"t={t}")
    layer.close()


SMALL = [
    small_config(901, L=3, d=64, M=200, K=96, C=8, mode="union", m=40, swap=6, T=8),
    small_config(902, L=2, d=200, M=1000, K=333, C=6, mode="union", m=150, swap=20, T=8),
    small_config(903, L=2, d=1000, M=130, K=50, C=5, mode="intersect", m=40, swap=8, T=8),
    small_config(904, L=2, d=4096, M=700, K=300, C=5, mode="single", R=2, m=250, swap=40, T=8),
    small_config(905, L=2, d=5120, M=640, K=256, C=4, mode="union", m=100, swap=20, T=6),
    small_config(906, L=2, d=7168, M=1100, K=700, C=4, mode="union", m=300, swap=50, T=6),
    small_config(907, L=1, d=8, M=64, K=64, C=3, mode="union", m=20, swap=4, T=6),
    # SwiGLU (SiLU gate) with intersected masks, as in the paper's models; and SiLU non-gated
    small_config(908, L=2, d=4096, M=1400, K=600, C=5, mode="intersect", m=600, swap=50, T=8, act="silu"),
    small_config(909, L=2, d=1000, M=500, K=200, C=4, mode="union", m=90, swap=12, T=6, act="silu"),
    small_config(910, L=2, d=512, M=300, K=120, C=4, mode="single", R=2, m=100, swap=10, T=6, act="silu"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"d{c.d}_M{c.M}_K{c.K}_{c.mode}_R{c.R}_{c.act}")
@pytest.mark.parametrize("streams,graphs", [(1, True), (1, False), (2, True), (2, False)])
def test_small_shapes_decode_step(torch, cfg, streams, graphs):
    from delta_prefetched_ffn_amd import binding as B
    B.decode_use_graphs(graphs)
    wl = Workload(cfg)
    layers, stores = zip(*[make_layer(wl, l) for l in range(cfg.L)])
    orc = OracleRun(wl)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    cs = torch.cuda.Stream()
    ps = torch.cuda.Stream() if streams == 2 else cs
    for t in range(cfg.T):
        B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), cs.cuda_stream, ps.cuda_stream)
        for l, layer in enumerate(layers):
            st = layer.read_state()
            S, res = orc.step(t, l, stores[l])
            compare_state(st, orc.layers[l], res, S, f"t={t} l={l}")
            assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"t={t} l={l}: buffer"
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    orc2 = OracleRun(wl, keep_buffer=False)
    for t in range(cfg.T):
        for l in range(cfg.L):
            S = orc2.active(t, l)
            check_y(yh[t, l], O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act), f"t={t} l={l}")
    for layer in layers:
        layer.close()
    B.decode_use_graphs(False)  # the library default


def _dyadic_store(rng, M, R, d):
    """Gate/up rows: 8 nonzeros in {+-1,+-2}/64; down rows: dense {-2..2}/64. Exact in bf16."""
    w = np.zeros((M, R, d), dtype=np.float32)
    for n in range(M):
        for r in range(R - 1):
            cols = rng.choice(d, size=8, replace=False)
            w[n, r, cols] = rng.choice([-2, -1, 1, 2], size=8) / 64.0
        w[n, R - 1] = rng.integers(-2, 3, size=d) / 64.0
    return (w.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("R", [3, 2])
def test_exact_dyadic_inputs_bit_exact(torch, R):
    """Every partial sum is a dyadic rational below 2^24 units: fp32 is exact in any order."""
    from delta_prefetched_ffn_amd import binding as B
    rng = np.random.default_rng(40 + R)
    M, d, K = 512, 4096, 256
    store = _dyadic_store(rng, M, R, d)
    mode = "union" if R == 3 else "single"
    cfg = Config(950 + R, "dyadic", L=1, d=d, M=M, R=R, K=K, C=4, mode=mode, T=4, m=100, swap=10)
    wl = Workload(cfg)
    layer, _ = make_layer(wl, 0, store=store)
    orc = OracleRun(wl, keep_buffer=False)
    s = _stream(torch)
    for t in range(cfg.T):
        x_np = (rng.integers(-8, 9, size=d) / 8.0).astype(np.float32)
        x = torch.from_numpy(x_np).cuda()
        y = torch.empty_like(x)
        g, u = (int(v) for v in wl.cids()[t, 0])
        layer.delta_assign(g, u, s)
        layer.scatter_rows(s)
        layer.sparse_ffn(x.data_ptr(), y.data_ptr(), s)
        S = orc.active(t, 0)
        assert S.size <= 256
        ref = O.sparse_ffn(store, R, d, S, x_np)
        got = y.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), f"t={t}: max diff {np.abs(got - ref).max()}"
    layer.close()


def test_decode_paths_agree_and_repeat_bitwise(torch):
    """With the ordered reduction: graph replay and direct launches, one stream and two streams,
    device, pinned-host and mixed row stores (with host stores each FFN launch also scatters the
    next layer's new bundles; mixed: a device-store layer between two host-store layers, whose
    FFN reads through and carries the prefetch), and per-layer calls give bit-identical y and
    slot buffers; reruns too."""
    from delta_prefetched_ffn_amd import binding as B
    cfg = small_config(960, L=3, d=4096, M=3000, K=600, C=6, mode="union", m=250, swap=30, T=6)
    wl = Workload(cfg)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    outs, bufs = [], []
    for path in ["two", "one", "calls", "calls-rt", "two-direct", "one-direct", "two-host", "two-host-direct",
                 "one-host", "one-host-direct", "two-mixed", "two-mixed-direct", "two"]:
        B.decode_use_graphs(not path.endswith("direct"))
        where = ["host" if "host" in path or ("mixed" in path and l != 1) else "device" for l in range(cfg.L)]
        layers = [make_layer(wl, l, where[l])[0] for l in range(cfg.L)]
        for layer in layers:
            layer.set_ffn_reduce("ordered")  # bit-identical results need the fixed-order reduction
        y = torch.zeros_like(x)
        cs, ps = torch.cuda.Stream(), torch.cuda.Stream()
        for t in range(cfg.T):
            if path.startswith("calls"):
                for l, layer in enumerate(layers):
                    g, u = (int(v) for v in wl.cids()[t, l])
                    layer.delta_assign(g, u, cs.cuda_stream)
                    if path == "calls":  # else the FFN reads the new bundles through
                        layer.scatter_rows(cs.cuda_stream)
                    layer.sparse_ffn(x[t, l].data_ptr(), y[t, l].data_ptr(), cs.cuda_stream)
            else:
                B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), cs.cuda_stream,
                              (ps if path.startswith("two") else cs).cuda_stream)
        torch.cuda.synchronize()
        assert all(L.read_state()["err"] == 0 for L in layers)
        outs.append(y.cpu().numpy())
        bufs.append(layers[-1].read_rows())
        for layer in layers:
            layer.close()
    B.decode_use_graphs(False)  # the library default
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    for b in bufs[1:]:  # slot buffers, stale rows included
        assert np.array_equal(b, bufs[0])


@pytest.mark.parametrize("reduce", ["ordered", "atomic"])
def test_token_launch_groups_graphs_and_fallback(torch, reduce):
    """Pinned-host row stores: a decode step runs as one launch per group of up to 64 layers
    (prefetch workgroups stream every layer's delta, each layer's FFN starts once its delta is
    in place). 70 layers take two launches per step. Against the oracle for every (step, layer):
    direct launches, graph replay, and (ordered reduction) bit-identical y and slot buffers in
    the two, and in per-layer calls. A layer with another FFN workgroup size makes the step
    fall back to per-layer launches, with the same results."""
    from delta_prefetched_ffn_amd import binding as B
    cfg = small_config(980, L=70, d=64, M=256, K=96, C=5, mode="union", m=60, swap=12, T=5)
    wl = Workload(cfg)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    orc = OracleRun(wl)
    stores = [wl.store(l) for l in range(cfg.L)]
    ref = {}
    for t in range(cfg.T):
        for l in range(cfg.L):
            S, _ = orc.step(t, l, stores[l])
            ref[t, l] = O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act)
    final_bufs = [orc.layers[l].buf.copy() for l in range(cfg.L)]
    outs = {}
    for path in ["token-direct", "token-graph", "calls", "fallback-direct", "fallback-calls"]:
        B.decode_use_graphs(path == "token-graph")
        layers = [make_layer(wl, l, "host", stores[l])[0] for l in range(cfg.L)]
        for layer in layers:
            layer.set_ffn_reduce(reduce)
        if path.startswith("fallback"):
            layers[33].set_ffn_shape(threads=512)  # the others use 256-thread workgroups at d = 64
        y = torch.zeros_like(x)
        s = torch.cuda.Stream()
        for t in range(cfg.T):
            if path.endswith("calls"):
                for l, layer in enumerate(layers):
                    g, u = (int(v) for v in wl.cids()[t, l])
                    layer.delta_assign(g, u, s.cuda_stream)
                    layer.scatter_rows(s.cuda_stream)
                    layer.sparse_ffn(x[t, l].data_ptr(), y[t, l].data_ptr(), s.cuda_stream)
            else:
                B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), s.cuda_stream, s.cuda_stream)
        torch.cuda.synchronize()
        assert all(L.read_state()["err"] == 0 for L in layers), path
        yh = y.cpu().numpy()
        for t in range(cfg.T):
            for l in range(cfg.L):
                check_y(yh[t, l], ref[t, l], f"{path} t={t} l={l}")
        for l in (0, 33, 63, 64, 69):
            assert np.array_equal(layers[l].read_rows(), final_bufs[l]), f"{path}: layer {l} buffer"
        outs[path] = yh
        for layer in layers:
            layer.close()
    B.decode_use_graphs(False)
    if reduce == "ordered":
        for a, b in (("token-graph", "token-direct"), ("calls", "token-direct"), ("fallback-calls", "fallback-direct")):
            assert np.array_equal(outs[a].view(np.uint32), outs[b].view(np.uint32)), (a, b)


def test_edge_cases_empty_full_turnover_and_exact_capacity(torch):
    from delta_prefetched_ffn_amd import binding as B
    M, K, d, R = 256, 64, 128, 3
    W = M // 64

    def mask(ids):
        m = np.zeros(M, dtype=bool)
        m[list(ids)] = True
        return np.packbits(m.astype(np.uint8), bitorder="little").view("<u8").astype(np.uint64)

    sets = [[], list(range(0, 64)), list(range(0, 64)), list(range(64, 128)), list(range(100, 140)), [],
            list(range(192, 256))]
    gate = np.stack([mask(s) for s in sets])
    up = np.stack([mask([]) for _ in sets])
    masks = np.stack([gate, up])
    rng = np.random.default_rng(3)
    store = ((rng.standard_normal((M, R, d)).astype(np.float32) * 0.02).view(np.uint32) >> 16).astype(np.uint16)
    dev = upload_store(store, "device")
    layer = B.Layer(d_model=d, d_ff=M, k_max=K, n_rows=R, masks=masks, mask_mode=B.MASK_UNION,
                    row_store=dev.data_ptr(), keepalive=dev)
    ol = O.OracleLayer(M, K, R, d)
    s = _stream(torch)
    x_np = rng.standard_normal(d).astype(np.float32)
    x = torch.from_numpy(x_np).cuda()
    for i, S_ids in enumerate(sets):
        y = torch.full((d,), float("nan"), device="cuda")
        layer.delta_assign(i, i, s)
        layer.scatter_rows(s)
        layer.sparse_ffn(x.data_ptr(), y.data_ptr(), s)
        st = layer.read_state()
        S = np.array(S_ids, dtype=np.int32)
        res = ol.step(S)
        ol.copy_bundles(store, res)
        compare_state(st, ol, res, S, f"step {i}")
        assert np.array_equal(layer.read_rows(), ol.buf)
        yh = y.cpu().numpy()
        if not S_ids:
            assert (yh == 0).all()
        check_y(yh, O.sparse_ffn(store, R, d, S, x_np), f"step {i}")
    layer.close()


def test_token_launch_edge_cases(torch):
    """The edge sequence above through np_decode_step on pinned host stores (the token launch),
    two layers whose sets differ, with every state, buffer and y checked: empty sets (no FFN
    work, no delta), |S| = K_max, full turnover, empty deltas for one layer while the other
    layer's delta is whole."""
    from delta_prefetched_ffn_amd import binding as B
    M, K, d, R = 256, 64, 128, 3
    W = M // 64

    def mask(ids):
        m = np.zeros(M, dtype=bool)
        m[list(ids)] = True
        return np.packbits(m.astype(np.uint8), bitorder="little").view("<u8").astype(np.uint64)

    seqs = [
        [[], list(range(0, 64)), list(range(0, 64)), list(range(64, 128)), list(range(100, 140)), [],
         list(range(192, 256))],
        [list(range(10, 20)), [], list(range(0, 64)), list(range(0, 64)), [], list(range(128, 192)),
         list(range(128, 192))],
    ]
    rng = np.random.default_rng(5)
    stores, layers, ols = [], [], []
    for l, sets in enumerate(seqs):
        gate = np.stack([mask(s_) for s_ in sets])
        up = np.stack([mask([]) for _ in sets])
        store = ((rng.standard_normal((M, R, d)).astype(np.float32) * 0.02).view(np.uint32) >> 16).astype(np.uint16)
        pinned = upload_store(store, "host")
        layers.append(B.Layer(d_model=d, d_ff=M, k_max=K, n_rows=R, masks=np.stack([gate, up]),
                              mask_mode=B.MASK_UNION, row_store=pinned.data_ptr(), keepalive=pinned))
        stores.append(store)
        ols.append(O.OracleLayer(M, K, R, d))
    s = torch.cuda.Stream()
    x_np = rng.standard_normal((2, d)).astype(np.float32)
    x = torch.from_numpy(x_np).cuda()
    for i in range(len(seqs[0])):
        y = torch.full((2, d), float("nan"), device="cuda")
        cids = np.array([[i, i], [i, i]], dtype=np.int32)
        B.decode_step(layers, cids, x.data_ptr(), y.data_ptr(), s.cuda_stream, s.cuda_stream)
        s.synchronize()
        yh = y.cpu().numpy()
        for l in range(2):
            S = np.array(seqs[l][i], dtype=np.int32)
            res = ols[l].step(S)
            ols[l].copy_bundles(stores[l], res)
            compare_state(layers[l].read_state(), ols[l], res, S, f"step {i} layer {l}")
            assert np.array_equal(layers[l].read_rows(), ols[l].buf), f"step {i} layer {l}: buffer"
            if S.size == 0:
                assert (yh[l] == 0).all(), f"step {i} layer {l}"
            check_y(yh[l], O.sparse_ffn(stores[l], R, d, S, x_np[l]), f"step {i} layer {l}")
    for layer in layers:
        layer.close()


def test_token_launch_layers_of_different_shapes(torch):
    """One decode step over layers that share d_model but differ in d_ff, K_max, mask mode and
    activation (pinned host stores: one token launch with per-layer shapes, deltas and FFN
    arguments), against the oracle at every (step, layer), and bit-identical to per-layer calls."""
    from delta_prefetched_ffn_amd import binding as B
    cfgs = [small_config(990, L=1, d=512, M=900, K=300, C=5, mode="union", m=120, swap=20, T=6),
            small_config(991, L=1, d=512, M=500, K=120, C=4, mode="intersect", m=100, swap=15, T=6, act="silu"),
            small_config(992, L=1, d=512, M=1300, K=500, C=6, mode="union", m=200, swap=40, T=6)]
    wls = [Workload(c) for c in cfgs]
    T = cfgs[0].T
    x_np = np.stack([np.concatenate([w.x_all()[t] for w in wls]) for t in range(T)])  # [T][3][d]
    x = torch.from_numpy(x_np).cuda()
    outs = {}
    for path in ["token", "calls"]:
        layers, stores = [], []
        for w in wls:
            layer, store = make_layer(w, 0, "host")
            layer.set_ffn_reduce("ordered")
            layers.append(layer)
            stores.append(store)
        orcs = [OracleRun(w) for w in wls]
        y = torch.zeros_like(x)
        s = torch.cuda.Stream()
        for t in range(T):
            cids = np.concatenate([w.cids()[t] for w in wls])
            if path == "token":
                B.decode_step(layers, cids, x[t].data_ptr(), y[t].data_ptr(), s.cuda_stream, s.cuda_stream)
            else:
                for l, layer in enumerate(layers):
                    layer.delta_assign(int(cids[l, 0]), int(cids[l, 1]), s.cuda_stream)
                    layer.scatter_rows(s.cuda_stream)
                    layer.sparse_ffn(x[t, l].data_ptr(), y[t, l].data_ptr(), s.cuda_stream)
            s.synchronize()
            for l, (w, orc) in enumerate(zip(wls, orcs)):
                S, res = orc.step(t, 0, stores[l])
                compare_state(layers[l].read_state(), orc.layers[0], res, S, f"{path} t={t} l={l}")
                check_y(y[t, l].cpu().numpy(), O.sparse_ffn(stores[l], w.cfg.R, w.cfg.d, S, x_np[t, l], w.cfg.act),
                        f"{path} t={t} l={l}")
        for l, orc in enumerate(orcs):
            assert np.array_equal(layers[l].read_rows(), orc.layers[0].buf), f"{path} layer {l}: buffer"
        outs[path] = y.cpu().numpy()
        for layer in layers:
            layer.close()
    assert np.array_equal(outs["token"].view(np.uint32), outs["calls"].view(np.uint32))


LIMITS = [
    # the largest d_model (16384: 512-thread FFN workgroups, four x chunks per lane, 64 tiles)
    small_config(970, L=1, d=16384, M=320, K=200, C=4, mode="union", m=90, swap=10, T=5),
    # the largest d_ff and k_max (65536; owner table far beyond the per-thread preload) with
    # the smallest d_model, |S| of tens of thousands, ragged last words nowhere
    small_config(971, L=1, d=8, M=65536, K=65536, C=3, mode="union", m=30000, swap=3000, T=4),
    # d_ff and k_max just under the limit with ragged words, non-gated SiLU
    small_config(972, L=1, d=24, M=65535, K=60001, C=3, mode="single", R=2, m=50000, swap=5000, T=4, act="silu"),
    # one neuron, one slot
    small_config(973, L=1, d=8, M=1, K=1, C=2, mode="union", m=1, swap=0, T=4),
]


@pytest.mark.parametrize("cfg", LIMITS, ids=lambda c: f"d{c.d}_M{c.M}_K{c.K}_{c.mode}_R{c.R}")
def test_maximum_and_minimum_sizes(torch, cfg):
    """The documented size limits and the degenerate one-neuron layer, through np_decode_step:
    state and buffer bit-exact, y in tolerance."""
    from delta_prefetched_ffn_amd import binding as B
    print(f"[limits] d={cfg.d} M={cfg.M} K={cfg.K}", flush=True)
    wl = Workload(cfg)
    layers, stores = zip(*[make_layer(wl, l) for l in range(cfg.L)])
    orc = OracleRun(wl)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    s = _stream(torch)
    for t in range(cfg.T):
        B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), s, s)
        for l, layer in enumerate(layers):
            st = layer.read_state()
            S, res = orc.step(t, l, stores[l])
            compare_state(st, orc.layers[l], res, S, f"t={t} l={l}")
            assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"t={t} l={l}: buffer"
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for t in range(cfg.T):
        for l in range(cfg.L):
            S = orc.active(t, l)
            check_y(yh[t, l], O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act), f"t={t} l={l}")
    for layer in layers:
        layer.close()


@pytest.mark.parametrize("shape", [(3, 128, 256), (5, 256, 512), (5, 256, 1024), (2, 64, 1024), (8, 128, 512),
                                   (16, 256, 256), (1, 256, 256), (4, 512, 512), (4, 1024, 1024), (6, 512, 1024)])
def test_ffn_launch_shapes(torch, shape):
    """Every launch shape gives the oracle's y (tolerance) and exact results on dyadic inputs."""
    from delta_prefetched_ffn_amd import binding as B
    spw, tw, nt = shape
    cfg = small_config(970, L=1, d=4096, M=2000, K=900, C=4, mode="union", m=300, swap=40, T=3)
    wl = Workload(cfg)
    layer, store = make_layer(wl, 0)
    layer.set_ffn_shape(spw, tw, nt)
    orc = OracleRun(wl, keep_buffer=False)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    s = _stream(torch)
    for t in range(cfg.T):
        g, u = (int(v) for v in wl.cids()[t, 0])
        layer.delta_assign(g, u, s)
        layer.scatter_rows(s)
        layer.sparse_ffn(x[t, 0].data_ptr(), y[t, 0].data_ptr(), s)
        assert layer.read_state()["err"] == 0
        S = orc.active(t, 0)
        check_y(y[t, 0].cpu().numpy(), O.sparse_ffn(store, cfg.R, cfg.d, S, x_all[t, 0], cfg.act), f"{shape} t={t}")
    layer.close()
    # exact arithmetic in the same shape
    rng = np.random.default_rng(77)
    dstore = _dyadic_store(rng, 512, 3, 4096)
    dcfg = Config(980, "dyadic", L=1, d=4096, M=512, R=3, K=256, C=4, mode="union", T=2, m=100, swap=10)
    dwl = Workload(dcfg)
    dl, _ = make_layer(dwl, 0, store=dstore)
    dl.set_ffn_shape(spw, tw, nt)
    dorc = OracleRun(dwl, keep_buffer=False)
    for t in range(dcfg.T):
        x_np = (rng.integers(-8, 9, size=4096) / 8.0).astype(np.float32)
        xd = torch.from_numpy(x_np).cuda()
        yd = torch.empty_like(xd)
        g, u = (int(v) for v in dwl.cids()[t, 0])
        dl.delta_assign(g, u, s)
        dl.scatter_rows(s)
        dl.sparse_ffn(xd.data_ptr(), yd.data_ptr(), s)
        ref = O.sparse_ffn(dstore, 3, 4096, dorc.active(t, 0), x_np)
        assert np.array_equal(yd.cpu().numpy().astype(np.float64), ref), f"{shape} t={t}"
    dl.close()


@pytest.mark.parametrize("mode", ["atomic", "ordered"])
def test_accumulate_and_reduce_modes(torch, mode):
    """np_sparse_ffn_acc adds the FFN output to y; np_sparse_ffn replaces y (also when y holds
    NaN); both reductions match the oracle; the ordered one repeats bit for bit."""
    from delta_prefetched_ffn_amd import binding as B
    cfg = small_config(980, L=1, d=4096, M=1200, K=500, C=4, mode="union", m=200, swap=30, T=4, act="silu")
    wl = Workload(cfg)
    layer, store = make_layer(wl, 0)
    layer.set_ffn_reduce(mode)
    orc = OracleRun(wl)
    x_all = wl.x_all()
    rng = np.random.default_rng(1)
    s = _stream(torch)
    for t in range(cfg.T):
        g, u = (int(v) for v in wl.cids()[t, 0])
        layer.delta_assign(g, u, s)
        S, res = orc.step(t, 0, store)
        x = torch.from_numpy(x_all[t, 0]).cuda()
        base = rng.standard_normal(cfg.d).astype(np.float32)
        y_acc = torch.from_numpy(base).cuda()
        y_new = torch.full((cfg.d,), float("nan"), device="cuda")
        layer.sparse_ffn_acc(x.data_ptr(), y_acc.data_ptr(), s)   # read-through on the first call
        layer.sparse_ffn(x.data_ptr(), y_new.data_ptr(), s)
        y_rep = torch.full((cfg.d,), float("nan"), device="cuda")
        layer.sparse_ffn(x.data_ptr(), y_rep.data_ptr(), s)
        torch.cuda.synchronize()
        ref = O.sparse_ffn(store, cfg.R, cfg.d, S, x_all[t, 0], cfg.act)
        check_y(y_new.cpu().numpy(), ref, f"{mode} t={t} replace")
        check_y(y_acc.cpu().numpy() - base, ref, f"{mode} t={t} accumulate")
        if mode == "ordered":
            assert np.array_equal(y_new.cpu().numpy().view(np.uint32), y_rep.cpu().numpy().view(np.uint32))
        compare_state(layer.read_state(), orc.layers[0], res, S, f"{mode} t={t}")
    layer.close()
