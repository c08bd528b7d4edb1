"""GPU parity of the staged delta I/O (NeuroPrefetcher section 3.5: host gather of the sorted
incoming rows into bounded pinned staging, DMA copy, device scatter, chunked when the delta
exceeds the staging), for row stores in pinned host memory: delta lists, slot map, owner table
and the whole buffer bit-exact against the oracle, y within max-abs 2e-2 / relative L2 5e-3,
on one and two streams, with staging small enough to force many chunks, for the slot and the
compacted layouts; layers with a window keep the zero-copy pull."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, compare_state, make_layer, torch_mod
from workload.gen import Workload, small_config

pytestmark = pytest.mark.gpu

SHAPES = [
    small_config(960, L=2, d=512, M=600, K=150, C=6, mode="union", m=60, swap=10, T=10),
    small_config(961, L=3, d=4096, M=1500, K=500, C=5, mode="union", m=200, swap=30, T=8),
    small_config(962, L=2, d=512, M=300, K=120, C=4, mode="single", R=2, m=100, swap=10, T=8, act="silu"),
]


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available()
    yield t
    from delta_prefetched_ffn_amd import binding as B
    B.decode_set_staging(0)  # the library default


@pytest.mark.parametrize("layout", ["slots", "compact"])
@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("per_chunk", [3, 1000])
@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: f"d{c.d}_M{c.M}_K{c.K}_{c.mode}_R{c.R}")
def test_staged_parity(torch, cfg, per_chunk, streams, layout):
    from delta_prefetched_ffn_amd import binding as B
    print(f"[staged] {cfg.num} chunk={per_chunk} streams={streams} {layout}", flush=True)
    B.decode_set_staging(per_chunk * cfg.bundle_bytes, 3)
    wl = Workload(cfg)
    layers, stores = zip(*[make_layer(wl, l, "host") for l in range(cfg.L)])
    for layer in layers:
        layer.set_layout(layout)
    orc = OracleRun(wl, layout=layout)
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
            what = f"t={t} l={l}"
            compare_state(st, orc.layers[l], res, S, what)
            assert np.array_equal(layer.read_rows(), orc.layers[l].buf), f"{what}: buffer"
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for t in range(cfg.T):
        for l in range(cfg.L):
            S = orc.active(t, l)
            check_y(yh[t, l], O.sparse_ffn(stores[l], cfg.R, cfg.d, S, x_all[t, l], cfg.act), f"t={t} l={l}")
    for layer in layers:
        layer.close()
    B.decode_set_staging(0)


def test_staged_with_a_window_layer_falls_back_to_the_pull(torch):
    from delta_prefetched_ffn_amd import binding as B
    cfg = SHAPES[0]
    B.decode_set_staging(4 * cfg.bundle_bytes)
    wl = Workload(cfg)
    layers, stores = zip(*[make_layer(wl, l, "host") for l in range(cfg.L)])
    layers[1].set_window(3)
    orcs = [OracleRun(wl), OracleRun(wl, window=3)]
    x = torch.from_numpy(wl.x_all()).cuda()
    y = torch.zeros_like(x)
    cs, ps = torch.cuda.Stream(), torch.cuda.Stream()
    for t in range(cfg.T):
        B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), cs.cuda_stream, ps.cuda_stream)
        for l, layer in enumerate(layers):
            S, res = orcs[l].step(t, l, stores[l])
            compare_state(layer.read_state(), orcs[l].layers[l], res, S, f"t={t} l={l}")
            assert np.array_equal(layer.read_rows(), orcs[l].layers[l].buf), f"t={t} l={l}: buffer"
    for layer in layers:
        layer.close()
    B.decode_set_staging(0)


def test_staging_checks(torch):
    from delta_prefetched_ffn_amd import binding as B
    for nbytes, threads in ((-1, 0), ((1 << 30) + 1, 0), (1 << 20, -1), (1 << 20, 65)):
        with pytest.raises(B.NPError) as e:
            B.decode_set_staging(nbytes, threads)
        assert e.value.status == B.NP_EINVAL
    cfg = SHAPES[1]
    B.decode_set_staging(cfg.bundle_bytes - 16)  # too small for one bundle
    wl = Workload(cfg)
    layers = [make_layer(wl, l, "host")[0] for l in range(cfg.L)]
    x = torch.zeros((cfg.L, cfg.d), dtype=torch.float32, device="cuda")
    y = torch.zeros_like(x)
    with pytest.raises(B.NPError) as e:
        B.decode_step(layers, wl.cids()[0], x.data_ptr(), y.data_ptr(), 0, 0)
    assert e.value.status == B.NP_EINVAL
    torch.cuda.synchronize()
    for layer in layers:
        layer.close()
    B.decode_set_staging(0)
