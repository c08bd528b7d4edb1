"""Host-side validation of the C ABI on a GPU: errors are synchronous and leave state unchanged."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.harness import compare_state, torch_mod, upload_store

pytestmark = pytest.mark.gpu

M, K, d, R = 512, 64, 64, 3


def _masks(sets_g, sets_u):
    def mask(ids):
        m = np.zeros(M, dtype=np.uint8)
        m[list(ids)] = 1
        return np.packbits(m, bitorder="little").view("<u8").astype(np.uint64)
    return np.stack([np.stack([mask(s) for s in sets_g]), np.stack([mask(s) for s in sets_u])])


@pytest.fixture
def env():
    torch = torch_mod()
    assert torch.cuda.is_available()
    from delta_prefetched_ffn_amd import binding as B
    rng = np.random.default_rng(0)
    store = ((rng.standard_normal((M, R, d)).astype(np.float32) * 0.02).view(np.uint32) >> 16).astype(np.uint16)
    dev = upload_store(store, "device")
    masks = _masks([range(0, 40), range(30, 70), range(0, 60)], [range(40, 64), range(100, 110), range(60, 70)])
    layer = B.Layer(d_model=d, d_ff=M, k_max=K, n_rows=R, masks=masks, mask_mode=B.MASK_UNION,
                    row_store=dev.data_ptr(), keepalive=dev)
    yield torch, B, layer, store, masks, dev
    layer.close()


def test_cid_range_capacity_and_order(env):
    torch, B, layer, store, masks, dev = env
    s = torch.cuda.current_stream().cuda_stream
    with pytest.raises(B.NPError) as e:
        layer.delta_assign(3, 0, s)
    assert e.value.status == B.NP_EINVAL
    with pytest.raises(B.NPError) as e:
        layer.delta_assign(0, -1, s)
    assert e.value.status == B.NP_EINVAL
    with pytest.raises(B.NPError) as e:
        layer.scatter_rows(s)                      # nothing assigned yet
    assert e.value.status == B.NP_ESTATE
    x = torch.zeros(d, device="cuda")
    y = torch.zeros(d, device="cuda")
    with pytest.raises(B.NPError) as e:
        layer.sparse_ffn(x.data_ptr(), y.data_ptr(), s)
    assert e.value.status == B.NP_ESTATE
    layer.delta_assign(0, 0, s)                    # |S| = 64 = K
    with pytest.raises(B.NPError) as e:
        layer.delta_assign(0, 0, s)                # assigned twice without scatter
    assert e.value.status == B.NP_ESTATE
    layer.scatter_rows(s)
    ol = O.OracleLayer(M, K, R, d)
    res = ol.step(np.arange(64, dtype=np.int32))
    st = layer.read_state()
    compare_state(st, ol, res, np.arange(64), "first")
    S1 = np.array(sorted(set(range(30, 70)) | set(range(100, 110))), dtype=np.int32)   # |S| = 50
    layer.delta_assign(1, 1, s)
    layer.scatter_rows(s)
    res1 = ol.step(S1)
    with pytest.raises(B.NPError) as e:
        layer.delta_assign(2, 2, s)                # |S| = 70 > K = 64
    assert e.value.status == B.NP_ECAPACITY
    st = layer.read_state()                        # unchanged by the refused call
    compare_state(st, ol, res1, S1, "after refusal")
    layer.sparse_ffn(x.data_ptr(), y.data_ptr(), s)  # the scattered state is still usable
    with pytest.raises(B.NPError) as e:
        layer.sparse_ffn(x.data_ptr() + 4, y.data_ptr(), s)
    assert e.value.status == B.NP_EINVAL


def test_decode_step_refusal_leaves_every_layer_unchanged(env):
    torch, B, layer, store, masks, dev = env
    layer2 = B.Layer(d_model=d, d_ff=M, k_max=K, n_rows=R, masks=masks, mask_mode=B.MASK_UNION,
                     row_store=dev.data_ptr(), keepalive=dev)
    x = torch.zeros((2, d), device="cuda")
    y = torch.zeros((2, d), device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    B.decode_step([layer, layer2], np.array([[0, 0], [1, 1]]), x.data_ptr(), y.data_ptr(), s, s)
    before = [layer.read_state(), layer2.read_state()]
    with pytest.raises(B.NPError) as e:
        B.decode_step([layer, layer2], np.array([[1, 1], [2, 2]]), x.data_ptr(), y.data_ptr(), s, s)
    assert e.value.status == B.NP_ECAPACITY
    after = [layer.read_state(), layer2.read_state()]
    for b, a in zip(before, after):
        for k in ("slot_map", "owner", "act"):
            assert np.array_equal(b[k], a[k])
    with pytest.raises(B.NPError) as e:
        B.decode_step([layer, layer], np.array([[1, 1], [1, 1]]), x.data_ptr(), y.data_ptr(), s, s)
    assert e.value.status == B.NP_EINVAL
    layer2.close()


def test_create_rejects_bad_descriptors(env):
    torch, B, layer, store, masks, dev = env
    kw = dict(d_model=d, d_ff=M, k_max=K, n_rows=R, masks=masks, mask_mode=B.MASK_UNION,
              row_store=dev.data_ptr())
    for bad in [dict(d_model=60), dict(k_max=M + 1), dict(n_rows=4), dict(mask_mode=7),
                dict(row_store=dev.data_ptr() + 2)]:
        with pytest.raises(B.NPError) as e:
            B.Layer(**{**kw, **bad})
        assert e.value.status == B.NP_EINVAL, bad
    pageable = np.zeros(M * R * d, dtype=np.uint16)
    with pytest.raises(B.NPError) as e:
        B.Layer(**{**kw, "row_store": pageable.ctypes.data})
    assert e.value.status == B.NP_EINVAL
    stray = _masks([[505], [1], [2]], [[3], [4], [5]])
    with pytest.raises(B.NPError) as e:      # neuron 505 is beyond d_ff = 502
        B.Layer(**{**kw, "d_ff": M - 10, "k_max": K, "masks": stray})
    assert e.value.status == B.NP_EINVAL


def test_reset_gives_a_cold_start(env):
    torch, B, layer, store, masks, dev = env
    s = torch.cuda.current_stream().cuda_stream
    layer.delta_assign(1, 1, s)
    layer.scatter_rows(s)
    layer.reset()
    layer.delta_assign(0, 0, s)
    layer.scatter_rows(s)
    st = layer.read_state()
    assert st["slot_in"].tolist() == list(range(64))
    assert st["d_out"].size == 0


def test_read_through_needs_a_device_store(env):
    """np_sparse_ffn right after np_delta_assign reads the new bundles through only from a
    device-memory row store; with a pinned-host store it refuses (NP_ESTATE) and the layer
    still accepts np_scatter_rows."""
    torch, B, layer, store, masks, dev = env
    host = upload_store(store, "host")
    hl = B.Layer(d_model=d, d_ff=M, k_max=K, n_rows=R, masks=masks, mask_mode=B.MASK_UNION,
                 row_store=host.data_ptr(), keepalive=host)
    s = torch.cuda.current_stream().cuda_stream
    x = torch.ones(d, device="cuda")
    y = torch.zeros(d, device="cuda")
    hl.delta_assign(0, 0, s)
    with pytest.raises(B.NPError) as e:
        hl.sparse_ffn(x.data_ptr(), y.data_ptr(), s)
    assert e.value.status == B.NP_ESTATE
    hl.scatter_rows(s)
    hl.sparse_ffn(x.data_ptr(), y.data_ptr(), s)
    layer.delta_assign(0, 0, s)
    layer.sparse_ffn(x.data_ptr(), y.data_ptr(), s)      # read-through
    with pytest.raises(B.NPError) as e:
        layer.scatter_rows(s)                              # already in the buffer
    assert e.value.status == B.NP_ESTATE
    torch.cuda.synchronize()
    ol = O.OracleLayer(M, K, R, d)
    res = ol.step(np.arange(64, dtype=np.int32))
    ol.copy_bundles(store, res)
    for L in (hl, layer):
        compare_state(L.read_state(), ol, res, np.arange(64), "first")
        assert np.array_equal(L.read_rows(), ol.buf)
    hl.close()


def test_device_errors_are_refused_until_reset(env):
    """Error bits raised on the device (here by np_layer_raise_error, through the path a failing
    kernel takes) make every later enqueueing call of the layer fail with NP_EDEVICE before it
    enqueues anything; np_layer_read_state returns the bits; np_layer_reset clears them; another
    layer is not affected."""
    torch, B, layer, store, masks, dev = env
    other = B.Layer(d_model=d, d_ff=M, k_max=K, n_rows=R, masks=masks, mask_mode=B.MASK_UNION,
                    row_store=dev.data_ptr(), keepalive=dev)
    s = torch.cuda.current_stream().cuda_stream
    x = torch.ones(2, d, device="cuda")
    y = torch.zeros(2, d, device="cuda")
    layer.delta_assign(0, 0, s)
    layer.sparse_ffn(x[0].data_ptr(), y[0].data_ptr(), s)
    torch.cuda.synchronize()
    assert layer.read_state()["err"] == 0
    before = layer.read_state()
    layer.raise_error(8, s)
    torch.cuda.synchronize()
    for call in (lambda: layer.delta_assign(1, 1, s),
                 lambda: layer.sparse_ffn(x[0].data_ptr(), y[0].data_ptr(), s),
                 lambda: B.decode_step([other, layer], np.array([[1, 1], [1, 1]], dtype=np.int32),
                                       x.data_ptr(), y.data_ptr(), s, s)):
        with pytest.raises(B.NPError) as e:
            call()
        assert e.value.status == B.NP_EDEVICE and "0x8" in str(e.value)
    st = layer.read_state(check=False)
    assert st["err"] == 8
    for k in ("slot_map", "owner", "d_in", "slot_in", "d_out", "act"):
        assert np.array_equal(st[k], before[k]), k           # nothing was enqueued
    assert other.read_state()["err"] == 0 and other.info()["n_active"] == 0
    with pytest.raises(B.NPError) as e:
        layer.read_state()
    assert e.value.status == B.NP_EDEVICE
    with pytest.raises(B.NPError):
        layer.raise_error(0, s)
    layer.reset()
    assert layer.read_state()["err"] == 0
    layer.delta_assign(1, 1, s)
    layer.sparse_ffn(x[0].data_ptr(), y[0].data_ptr(), s)
    torch.cuda.synchronize()
    assert layer.read_state()["err"] == 0
    other.close()


def test_io_pointers_must_be_gpu_accessible(env):
    """x and y must be device memory of the layer's device or mapped pinned host memory: a
    pageable host pointer is refused on the host (NP_EINVAL) instead of faulting the GPU."""
    torch, B, layer, store, masks, dev = env
    s = torch.cuda.current_stream().cuda_stream
    layer.delta_assign(0, 0, s)
    layer.scatter_rows(s)
    raw = np.zeros(d + 64, dtype=np.float32)
    off = (-raw.ctypes.data % 64) // 4
    pageable = raw[off:off + d]
    assert pageable.ctypes.data % 16 == 0
    x = torch.ones(d, device="cuda")
    y = torch.zeros(d, device="cuda")
    for xp, yp, name in ((pageable.ctypes.data, y.data_ptr(), "x"), (x.data_ptr(), pageable.ctypes.data, "y")):
        with pytest.raises(B.NPError) as e:
            layer.sparse_ffn(xp, yp, s)
        assert e.value.status == B.NP_EINVAL and str(e.value).split(": ", 1)[1].startswith(name)
    with pytest.raises(B.NPError) as e:
        B.decode_step([layer], np.array([[1, 1]], dtype=np.int32), pageable.ctypes.data, y.data_ptr(), s, s)
    assert e.value.status == B.NP_EINVAL
    assert layer.info()["n_active"] > 0 and layer.read_state()["err"] == 0   # nothing was enqueued
    xh = torch.ones(d, dtype=torch.float32, pin_memory=True)               # mapped pinned host memory
    layer.sparse_ffn(xh.data_ptr(), y.data_ptr(), s)
    ref = y.clone()
    layer.sparse_ffn(x.data_ptr(), y.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.equal(ref, y) or torch.allclose(ref, y, rtol=0, atol=1e-6)
