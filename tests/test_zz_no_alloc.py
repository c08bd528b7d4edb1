"""np_sparse_ffn_noalloc (the FFN with its exchange words in the library's static scratch) against
np_sparse_ffn on the same layer state, through the C ABI: y bit-identical (both use the ordered
reduction) and within tolerance of the oracle, on two calls in a row, the second on a smaller
layer; a launch shape beyond the scratch is refused before anything is enqueued."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import OracleRun, check_y, make_layer, torch_mod
from workload.gen import Workload, small_config

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def test_noalloc_matches_sparse_ffn_on_two_calls():
    torch = torch_mod()
    assert torch.cuda.is_available()
    from delta_prefetched_ffn_amd import binding as B
    s = torch.cuda.Stream()
    big = small_config(2100, L=1, d=4096, M=11008, K=4096, C=4, mode="union", m=1130, swap=102, T=3)
    small = small_config(2101, L=1, d=1000, M=700, K=260, C=4, mode="intersect", m=200, swap=30, T=3, act="silu")
    for k, cfg in enumerate([big, small]):   # the second call: a smaller layer, a smaller launch
        wl = Workload(cfg)
        layer, store = make_layer(wl, 0)
        orc = OracleRun(wl)
        for t in range(cfg.T):
            g, u = (int(v) for v in wl.cids()[t, 0])
            layer.delta_assign(g, u, s.cuda_stream)
            S, res = orc.step(t, 0, store)
            x = torch.from_numpy(wl.x_all()[t, 0]).cuda()
            y_ref = torch.full((cfg.d,), float("nan"), device="cuda")
            y_na = torch.full((cfg.d,), float("nan"), device="cuda")
            if t % 2 == 0:   # the no-allocation call first (it then reads the new bundles through)
                layer.sparse_ffn_noalloc(x.data_ptr(), y_na.data_ptr(), s.cuda_stream)
                layer.sparse_ffn(x.data_ptr(), y_ref.data_ptr(), s.cuda_stream)
            else:
                layer.sparse_ffn(x.data_ptr(), y_ref.data_ptr(), s.cuda_stream)
                layer.sparse_ffn_noalloc(x.data_ptr(), y_na.data_ptr(), s.cuda_stream)
            s.synchronize()
            assert np.array_equal(_bits(y_na), _bits(y_ref)), f"call {k} t={t}: y differs from np_sparse_ffn"
            ref = O.sparse_ffn(store, cfg.R, cfg.d, S, wl.x_all()[t, 0], cfg.act)
            check_y(y_na.cpu().numpy(), ref, f"call {k} t={t}")
            st = layer.read_state()
            assert st["err"] == 0
            got = layer.read_rows(res.slot_in)
            assert np.array_equal(got, wl.bundles(0, res.d_in)), f"call {k} t={t}: read-through rows"
        layer.close()


def test_noalloc_refuses_a_launch_beyond_its_scratch():
    torch = torch_mod()
    assert torch.cuda.is_available()
    from delta_prefetched_ffn_amd import binding as B
    # d_model 16384 with 64-column tiles (256 tiles) and one slot per workgroup: about 3,300
    # workgroups x 64 partial words, more than the 196,608 the scratch holds.
    cfg = small_config(2102, L=1, d=16384, M=4096, K=4096, C=2, mode="single", m=3000, swap=10, T=1, R=2)
    wl = Workload(cfg)
    layer, store = make_layer(wl, 0)
    layer.set_ffn_shape(1, 64, 0)
    s = torch.cuda.Stream()
    g, u = (int(v) for v in wl.cids()[0, 0])
    layer.delta_assign(g, u, s.cuda_stream)
    x = torch.from_numpy(wl.x_all()[0, 0]).cuda()
    y = torch.full((cfg.d,), float("nan"), device="cuda")
    with pytest.raises(B.NPError) as e:
        layer.sparse_ffn_noalloc(x.data_ptr(), y.data_ptr(), s.cuda_stream)
    assert e.value.status == B.NP_EINVAL and "scratch" in str(e.value)
    s.synchronize()
    assert torch.isnan(y).all()                      # nothing was enqueued
    layer.sparse_ffn(x.data_ptr(), y.data_ptr(), s.cuda_stream)   # the allocating entry point serves it
    s.synchronize()
    S = O.active_set(wl.masks(0)[0][g], None, cfg.M, O.SINGLE)
    check_y(y.cpu().numpy(), O.sparse_ffn(store, cfg.R, cfg.d, S, wl.x_all()[0, 0], cfg.act), "fallback")
    layer.close()
