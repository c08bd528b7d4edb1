"""GPU parity over seeded random combinations of shape and options, each case against the
oracle at every step: small shapes of random d_model (one to 640 16-byte chunks per row,
across the 256/512/1024-thread launch shapes), d_ff, K_max, mask mode and row count, ReLU or
SiLU, crossed with one retention rule (exact S, a residency window, frequency levels or the
compacted layout), slot or planar buffers, atomic or ordered reduce, a random FFN launch shape
and one of four launch paths (np_decode_step with direct launches or graph replay, per-layer
np_delta_assign + read-through np_sparse_ffn, pinned-host store: the token launch). Each option
has its own tests elsewhere; this file looks for interactions between them.

Checked per (step, layer): delta lists, slot map, owner table and the FFN's slot list
bit-exact (plus the compacted positions and moves); the whole slot buffer, stale rows
included, bit-exact after the last step; y within max-abs 2e-2 / relative L2 5e-3."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, compare_state, make_layer, torch_mod
from workload.gen import Workload, small_config

N_CASES = 96


def draw_case(i: int) -> dict:
    """Case i of the sweep, from its own seed (reproducible, independent of the others)."""
    rng = np.random.default_rng(20261202 + 7919 * i)
    cpr = int(rng.choice([1, 3, 8, 40, 64, 125, 512, 640]))        # 16-byte chunks per row
    d = 8 * cpr
    gated = bool(rng.integers(0, 3) > 0)
    R = 3 if gated else 2
    mode = str(rng.choice(["union", "intersect"])) if gated else "single"
    M = int(rng.integers(40, 1500))
    m = int(rng.integers(4, max(5, M // 3)))
    swap = int(rng.integers(0, max(1, m // 4)))
    need = 2 * m if mode == "union" else m
    K = int(min(M, need + rng.integers(0, max(1, need // 2) + 1)))
    ret = str(rng.choice(["exact", "window", "levels", "compact"]))
    case = {
        "i": i, "d": d, "M": M, "K": K, "R": R, "mode": mode, "m": m, "swap": swap,
        "act": str(rng.choice(["relu", "silu"])),
        "C": int(rng.integers(2, 7)), "T": int(rng.integers(5, 9)),
        "ret": ret,
        "window": int(rng.choice([2, 3, 5])) if ret == "window" else 1,
        "levels": int(rng.choice([1, 3, 8])) if ret == "levels" else 0,
        "planar": bool(rng.integers(0, 2)),
        "reduce": str(rng.choice(["atomic", "ordered"])),
        "shape": (int(rng.choice([0, 0, -1, 2, 7])), int(rng.choice([0, 0, 64, 128, 256, 512])),
                  int(rng.choice([0, 0, 256, 512, 1024]))),
        "path": str(rng.choice(["direct", "graph", "calls", "host2"])),
    }
    return case


CASES = [draw_case(i) for i in range(N_CASES)]


def case_id(c: dict) -> str:
    return (f"{c['i']}-d{c['d']}-M{c['M']}-K{c['K']}-R{c['R']}-{c['mode']}-{c['act']}-{c['ret']}"
            f"{c['window'] if c['ret'] == 'window' else c['levels'] if c['ret'] == 'levels' else ''}"
            f"-{'planar' if c['planar'] else 'interleaved'}-{c['reduce']}-{c['path']}")


@pytest.fixture(scope="module")
def torch():  # GPU tests only
    t = torch_mod()
    assert t.cuda.is_available()
    return t


def test_sweep_covers_every_option():
    """The seeded draw reaches every value of every option at least once."""
    seen = {k: {str(c[k]) for c in CASES} for k in ("mode", "act", "ret", "planar", "reduce", "path")}
    assert seen["mode"] == {"union", "intersect", "single"}
    assert seen["act"] == {"relu", "silu"}
    assert seen["ret"] == {"exact", "window", "levels", "compact"}
    assert seen["planar"] == {"True", "False"}
    assert seen["reduce"] == {"atomic", "ordered"}
    assert seen["path"] == {"direct", "graph", "calls", "host2"}
    assert len({c["d"] for c in CASES}) >= 6


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_combination_parity(torch, case):
    from delta_prefetched_ffn_amd import binding as B
    print(f"[combo] {case_id(case)} shape={case['shape']}", flush=True)
    cfg = small_config(1300 + case["i"], L=2, d=case["d"], M=case["M"], R=case["R"], K=case["K"], C=case["C"],
                       mode=case["mode"], T=case["T"], m=case["m"], swap=case["swap"], act=case["act"])
    wl = Workload(cfg)
    path = case["path"]
    B.decode_use_graphs(path == "graph")
    where = "host" if path == "host2" else "device"
    layers, stores = zip(*[make_layer(wl, l, where) for l in range(cfg.L)])
    layout = "compact" if case["ret"] == "compact" else "slots"
    for l, layer in enumerate(layers):
        if case["window"] > 1:
            layer.set_window(case["window"])
        if case["levels"]:
            layer.set_levels(wl.frequency_levels(l, case["levels"]), case["levels"])
        if layout == "compact":
            layer.set_layout("compact")
        if case["planar"]:
            layer.set_planar(True)
        layer.set_ffn_reduce(case["reduce"])
        spw, tw, nt = case["shape"]
        if spw or tw or nt:
            try:
                layer.set_ffn_shape(spw, tw, nt)
            except B.NPError:
                pass  # a launch shape that cannot cover this k_max keeps the default one
    orc = OracleRun(wl, window=case["window"], n_levels=case["levels"], layout=layout)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    cs = torch.cuda.Stream()
    ps = torch.cuda.Stream() if path == "host2" else cs
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
            what = f"{case_id(case)} t={t} l={l}"
            compare_state(st, orc.layers[l], res, S, what)
            if layout == "compact":
                assert np.array_equal(st["act"], np.arange(S.size)), f"{what}: rows are not the prefix"
                src, dst = layer.read_moves()
                assert np.array_equal(src, res.mv_src) and np.array_equal(dst, res.mv_dst), f"{what}: moves"
    torch.cuda.synchronize()
    for l, layer in enumerate(layers):
        assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"{case_id(case)} l={l}: buffer"
    yh = y.cpu().numpy()
    for t in range(cfg.T):
        for l in range(cfg.L):
            S = orc.active(t, l)
            check_y(yh[t, l], O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act),
                    f"{case_id(case)} t={t} l={l}")
    for layer in layers:
        layer.close()
    B.decode_use_graphs(False)
