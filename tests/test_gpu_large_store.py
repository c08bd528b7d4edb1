"""GPU parity with a device row store above 4 GiB.

The FFN reads new bundles straight from a device row store through a buffer
descriptor with 32-bit offsets, so a store above 4 GiB is scattered into the
slots first. These tests place a 5.9 GB store in HBM (d_model 16384, d_ff
60000, three rows per bundle: neurons from 43691 up start beyond 4 GiB), run
np_sparse_ffn right after an assignment (no explicit scatter) and np_decode_step
on every decode path, and compare state, slot contents and y with the oracle.

Only the bundles the workload's masks can activate are written into the store
(the rest stay zero); the oracle's y takes those bundles, regenerated from the
same counter-based stream, as a compact store in the active set's order.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, compare_state, torch_mod
from workload.gen import small_config, Workload

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available(), "GPU tests need a visible GPU"
    from delta_prefetched_ffn_amd import binding
    binding.lib()  # fails loudly if the HIP library is missing
    return t


def _cfg(num, L, T):
    return small_config(num, L=L, d=16384, M=60000, K=256, C=4, mode="union", m=100, swap=20, T=T)


def _mask_members(wl: Workload, l: int) -> np.ndarray:
    """Every neuron any centroid mask of layer l holds (a superset of every active set)."""
    c = wl.cfg
    bits = np.unpackbits(wl.masks(l).view(np.uint8), axis=-1, bitorder="little")[..., : c.M]
    return np.flatnonzero(bits.reshape(-1, c.M).any(axis=0)).astype(np.int32)


def _big_layer(torch, wl: Workload, l: int):
    """A layer over a zeroed device store holding the bundles of its mask members."""
    from delta_prefetched_ffn_amd import binding as B
    c = wl.cfg
    assert c.M * c.bundle_bytes > FOUR_GIB
    ids = _mask_members(wl, l)
    assert int(ids.max()) * c.bundle_bytes >= FOUR_GIB, "no member lies beyond 4 GiB"
    store = torch.zeros((c.M, c.R * c.d), dtype=torch.int16, device="cuda")
    store[torch.from_numpy(ids.astype(np.int64)).cuda()] = \
        torch.from_numpy(wl.bundles(l, ids).reshape(ids.size, -1).view(np.int16)).cuda()
    layer = B.Layer(d_model=c.d, d_ff=c.M, k_max=c.K, n_rows=c.R, masks=wl.masks(l),
                    mask_mode=B.MODES[c.mode], act=B.ACTS[c.act], row_store=store.data_ptr(), keepalive=store)
    return layer


def _check_slots(wl: Workload, l: int, layer, st: dict, what: str) -> None:
    """Every active slot holds its owner's bundle, bit for bit."""
    act = st["act"]
    got = layer.read_rows(act)
    want = wl.bundles(l, st["owner"][act])
    assert np.array_equal(got, want), f"{what}: slot contents differ"


def _y_ref(wl: Workload, l: int, S: np.ndarray, x: np.ndarray) -> np.ndarray:
    c = wl.cfg
    return O.sparse_ffn(wl.bundles(l, S), c.R, c.d, np.arange(S.size, dtype=np.int32), x, c.act)


def test_large_store_single_layer_calls(torch):
    """np_delta_assign then np_sparse_ffn (and np_sparse_ffn_acc), without np_scatter_rows."""
    wl = Workload(_cfg(980, L=1, T=5))
    c = wl.cfg
    print(f"[large store] d={c.d} M={c.M} store={c.M * c.bundle_bytes / 1e9:.2f} GB", flush=True)
    layer = _big_layer(torch, wl, 0)
    orc = OracleRun(wl)
    x_all = wl.x_all()
    x = torch.from_numpy(x_all).cuda()
    y = torch.zeros_like(x)
    s = torch.cuda.current_stream().cuda_stream
    beyond = 0
    for t in range(c.T):
        g, u = (int(v) for v in wl.cids()[t, 0])
        layer.delta_assign(g, u, s)
        if t == c.T - 1:
            y[t, 0].copy_(x[t, 0])
            layer.sparse_ffn_acc(x[t, 0].data_ptr(), y[t, 0].data_ptr(), s)
        else:
            layer.sparse_ffn(x[t, 0].data_ptr(), y[t, 0].data_ptr(), s)
        st = layer.read_state()
        S, res = orc.step(t, 0)
        compare_state(st, orc.layers[0], res, S, f"t={t}")
        _check_slots(wl, 0, layer, st, f"t={t}")
        beyond += int((res.d_in.astype(np.int64) * c.bundle_bytes >= FOUR_GIB).sum())
        ref = _y_ref(wl, 0, S, x_all[t, 0])
        if t == c.T - 1:
            ref = ref + x_all[t, 0].astype(np.float64)
        check_y(y[t, 0].cpu().numpy(), ref, f"t={t}")
    assert beyond > 0, "no incoming bundle came from beyond 4 GiB"
    layer.close()


@pytest.mark.parametrize("streams,graphs", [(1, False), (1, True), (2, False)])
def test_large_store_decode_step(torch, streams, graphs):
    """np_decode_step over two layers with stores above 4 GiB, on one or two streams, with
    and without graph replay."""
    from delta_prefetched_ffn_amd import binding as B
    wl = Workload(_cfg(981, L=2, T=5))
    c = wl.cfg
    print(f"[large store decode] streams={streams} graphs={graphs}", flush=True)
    B.decode_use_graphs(graphs)
    try:
        layers = [_big_layer(torch, wl, l) for l in range(c.L)]
        orc = OracleRun(wl)
        x_all = wl.x_all()
        x = torch.from_numpy(x_all).cuda()
        y = torch.zeros_like(x)
        cs = torch.cuda.Stream()
        ps = torch.cuda.Stream() if streams == 2 else cs
        for t in range(c.T):
            B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), cs.cuda_stream, ps.cuda_stream)
            for l, layer in enumerate(layers):
                st = layer.read_state()
                S, res = orc.step(t, l)
                compare_state(st, orc.layers[l], res, S, f"t={t} l={l}")
                _check_slots(wl, l, layer, st, f"t={t} l={l}")
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        orc2 = OracleRun(wl, keep_buffer=False)
        for t in range(c.T):
            for l in range(c.L):
                S = orc2.active(t, l)
                check_y(yh[t, l], _y_ref(wl, l, S, x_all[t, l]), f"t={t} l={l}")
        for layer in layers:
            layer.close()
    finally:
        B.decode_use_graphs(False)  # the library default
