"""The measurement probes and the running counters: the copy probe moves exactly the bytes asked
for, the read probe touches every workgroup's sink entry, bad arguments are refused; the
counters (sum of |S| and of |D_in|) and np_layer_info equal the oracle's totals."""
import numpy as np
import pytest

from tests.harness import OracleRun, make_layer, torch_mod
from workload.gen import Workload, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    assert t.cuda.is_available()
    return t


def test_copy_probe_is_exact(torch):
    from delta_prefetched_ffn_amd import binding as B
    n = (1 << 20) + 48
    src = torch.randint(-32768, 32767, (n // 2,), dtype=torch.int16, device="cuda")
    dst = torch.zeros(n // 2 + 64, dtype=torch.int16, device="cuda")
    B.probe_copy(dst.data_ptr(), src.data_ptr(), n)
    torch.cuda.synchronize()
    assert torch.equal(dst[: n // 2], src) and (dst[n // 2:] == 0).all()


def test_read_probe_fills_its_sink(torch):
    from delta_prefetched_ffn_amd import binding as B
    n = 64 << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.full((65536,), float("nan"), dtype=torch.float32, device="cuda")
    B.probe_read(src.data_ptr(), n, sink.data_ptr())
    torch.cuda.synchronize()
    written = torch.isfinite(sink).sum().item()
    assert written > 0 and (sink[:written] >= 0).all()


def test_read_probe_set_reads_every_buffer(torch):
    from delta_prefetched_ffn_amd import binding as B
    n = 4 << 20
    bufs = [torch.ones(n // 4, dtype=torch.int32, device="cuda") for _ in range(3)]
    sink = torch.full((65536,), float("nan"), dtype=torch.float32, device="cuda")
    B.probe_read_set([b.data_ptr() for b in bufs], n, 2, sink.data_ptr())
    torch.cuda.synchronize()
    written = torch.isfinite(sink).sum().item()
    assert written > 0 and (sink[:written] >= 0).all()
    with pytest.raises(B.NPError):
        B.probe_read_set([], n, 1, sink.data_ptr())
    with pytest.raises(B.NPError):
        B.probe_read_set([bufs[0].data_ptr(), 0], n, 1, sink.data_ptr())
    with pytest.raises(B.NPError):
        B.probe_read_set([bufs[0].data_ptr() + 8], n, 1, sink.data_ptr())
    with pytest.raises(B.NPError):
        B.probe_read_set([bufs[0].data_ptr()], n + 8, 1, sink.data_ptr())
    with pytest.raises(B.NPError):
        B.probe_read_set([bufs[0].data_ptr()], n, 0, sink.data_ptr())


def test_probe_arguments_are_checked(torch):
    from delta_prefetched_ffn_amd import binding as B
    buf = torch.zeros(1 << 12, dtype=torch.int32, device="cuda")
    sink = torch.zeros(65536, dtype=torch.float32, device="cuda")
    p = buf.data_ptr()
    for args in ((p + 4, 1024), (p, 1000), (p, 0)):
        with pytest.raises(B.NPError) as e:
            B.probe_read(args[0], args[1], sink.data_ptr())
        assert e.value.status == B.NP_EINVAL
    with pytest.raises(B.NPError) as e:
        B.probe_copy(p + 8, p + 8192, 1024)
    assert e.value.status == B.NP_EINVAL


def test_counters_and_info_match_the_oracle(torch):
    from delta_prefetched_ffn_amd import binding as B
    cfg = small_config(990, L=3, d=256, M=700, K=200, C=5, mode="union", m=80, swap=12, T=9)
    wl = Workload(cfg)
    layers = [make_layer(wl, l)[0] for l in range(cfg.L)]
    orc = OracleRun(wl, keep_buffer=False)
    x = torch.from_numpy(wl.x_all()).cuda()
    y = torch.zeros_like(x)
    tot = np.zeros((cfg.L, 2), dtype=np.int64)
    for t in range(cfg.T):
        B.decode_step(layers, wl.cids()[t], x[t].data_ptr(), y[t].data_ptr(), 0, 0)
        for l, layer in enumerate(layers):
            S, res = orc.step(t, l)
            tot[l] += (S.size, res.d_in.size)
            info = layer.info()
            assert (info["n_active"], info["n_in"]) == (S.size, res.d_in.size), f"t={t} l={l}"
            assert (info["d_model"], info["d_ff"], info["k_max"], info["n_rows"]) == (cfg.d, cfg.M, cfg.K, cfg.R)
    torch.cuda.synchronize()
    for l, layer in enumerate(layers):
        assert tuple(layer.counters()) == tuple(tot[l]), f"layer {l}"
        layer.reset()
        assert tuple(layer.counters()) == (0, 0)
        layer.close()


def test_probe_pointers_must_be_gpu_accessible(torch):
    """A pageable host pointer given to a probe is refused on the host, before any launch."""
    from delta_prefetched_ffn_amd import binding as B
    raw = np.zeros((1 << 16) + 64, dtype=np.uint8)
    host = raw.ctypes.data + (-raw.ctypes.data % 64)
    dev = torch.zeros(1 << 14, dtype=torch.int32, device="cuda")
    sink = torch.zeros(65536, dtype=torch.float32, device="cuda")
    for call in (lambda: B.probe_read(host, 1 << 16, sink.data_ptr()),
                 lambda: B.probe_read(dev.data_ptr(), 1 << 16, host),
                 lambda: B.probe_read_set([dev.data_ptr(), host], 1 << 16, 1, sink.data_ptr()),
                 lambda: B.probe_copy(dev.data_ptr(), host, 1 << 16),
                 lambda: B.probe_copy(host, dev.data_ptr(), 1 << 16)):
        with pytest.raises(B.NPError) as e:
            call()
        assert e.value.status == B.NP_EINVAL
