"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU (no GPU needed).

Two builds made for this test only (under _build/san, rebuilt when a source is newer):
  * the oracle (oracle.c) compiled by clang with -fsanitize=address,undefined, UB reports fatal;
  * libnp with its host code compiled the same way (each -fsanitize= behind -Xarch_host; the gfx950
    device code is built as usual).
Each runs in a child process with the clang ASan runtime preloaded. The oracle build runs the
oracle's own pin tests; the libnp build is driven through every host-side check that runs before
any device call (descriptor limits, NULL and misaligned pointers, step arguments, staging and probe
bounds, error text), which needs no GPU. The checks that need a layer (centroid range, capacity,
call order) need a device to create one; tests/test_gpu_abi_errors.py covers them on the GPU.
A sanitizer report makes the child fail, and the report is in the assertion message.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "_build", "san")


def _runtime():
    sys.path.insert(0, ROOT)
    from delta_prefetched_ffn_amd.build import sanitizer_runtime
    rt = sanitizer_runtime()
    if not rt:
        pytest.skip("no clang ASan runtime in this image")
    return rt


def _env(extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime() + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    env["PYTHONPATH"] = ROOT
    env.update(extra)
    return env


def _run(cmd, env):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"exit {r.returncode}\n{out[-6000:]}"
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-6000:]
    return out


def test_oracle_pins_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from oracle.oracle import build_sanitized_lib
    lib = build_sanitized_lib(SAN_DIR)
    tests = [os.path.join("tests", f) for f in ("test_oracle_state.py", "test_oracle_ffn.py", "test_oracle_window.py",
                                                "test_oracle_levels.py", "test_oracle_compact.py")]
    out = _run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests],
               _env({"NPO_LIB": lib}))
    assert " passed" in out


def test_libnp_host_checks_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from delta_prefetched_ffn_amd.build import build_sanitized
    lib = build_sanitized()
    script = textwrap.dedent(r'''
        import ctypes, sys
        import numpy as np
        L = ctypes.CDLL(sys.argv[1])
        L.np_last_error.restype = ctypes.c_char_p
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        class Desc(ctypes.Structure):
            _fields_ = [(k, ctypes.c_int32) for k in ("d_model", "d_ff", "k_max", "n_rows", "n_centroids",
                        "mask_mode", "act", "device")] + [("masks", vp), ("row_store", vp)]
        EINVAL = 1
        masks = np.zeros(64, dtype=np.uint64)
        store = np.zeros(4096, dtype=np.uint16)
        good = dict(d_model=64, d_ff=128, k_max=32, n_rows=3, n_centroids=1, mask_mode=0, act=0, device=0)
        bad = [dict(d_model=0), dict(d_model=12), dict(d_model=16392), dict(d_ff=0), dict(d_ff=65537),
               dict(k_max=0), dict(k_max=129), dict(n_rows=1), dict(n_rows=4), dict(n_centroids=0),
               dict(n_centroids=65537), dict(mask_mode=3), dict(mask_mode=-1), dict(act=2),
               dict(d_model=16384, d_ff=65536, k_max=65536)]
        out = ctypes.c_void_p(123)
        for b in bad:
            d = Desc(**{**good, **b}, masks=masks.ctypes.data, row_store=store.ctypes.data)
            rc = L.np_layer_create(ctypes.byref(d), ctypes.byref(out))
            assert rc == EINVAL and out.value is None, (b, rc, L.np_last_error())
            assert L.np_last_error(), b
        d = Desc(**good, masks=None, row_store=store.ctypes.data)
        assert L.np_layer_create(ctypes.byref(d), ctypes.byref(out)) == EINVAL
        d = Desc(**good, masks=masks.ctypes.data, row_store=store.ctypes.data + 2)  # misaligned
        assert L.np_layer_create(ctypes.byref(d), ctypes.byref(out)) == EINVAL
        assert L.np_layer_create(None, None) == EINVAL
        # calls on a NULL layer
        for name, args in [("np_layer_destroy", [None]), ("np_layer_reset", [None]),
                           ("np_delta_assign", [None, 0, 0, None]), ("np_scatter_rows", [None, None]),
                           ("np_sparse_ffn", [None, None, None, None]), ("np_sparse_ffn_acc", [None, None, None, None]),
                           ("np_layer_set_ffn_reduce", [None, 1]), ("np_layer_set_ffn_shape", [None, 0, 0, 0]),
                           ("np_layer_set_window", [None, 2]), ("np_layer_set_levels", [None, 0, None]),
                           ("np_layer_set_layout", [None, 1]), ("np_layer_set_planar", [None, 1]),
                           ("np_layer_read_state", [None] * 8), ("np_layer_read_rows", [None, None, 0, None]),
                           ("np_layer_read_moves", [None] * 4), ("np_layer_info", [None, None]),
                           ("np_layer_counters", [None, None]), ("np_layer_raise_error", [None, 1, None])]:
            assert getattr(L, name)(*args) == EINVAL, name
        # decode step arguments, checked before any layer is touched
        x = np.zeros(64, dtype=np.float32)
        cids = np.zeros(2, dtype=np.int32)
        L.np_decode_step.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        assert L.np_decode_step(None, 1, cids.ctypes.data, x.ctypes.data, x.ctypes.data, None, None) == EINVAL
        handles = (ctypes.c_void_p * 1)(None)
        assert L.np_decode_step(handles, 0, cids.ctypes.data, x.ctypes.data, x.ctypes.data, None, None) == EINVAL
        assert L.np_decode_step(handles, 1, None, x.ctypes.data, x.ctypes.data, None, None) == EINVAL
        assert L.np_decode_step(handles, 1, cids.ctypes.data, x.ctypes.data + 4, x.ctypes.data, None, None) == EINVAL
        # process-wide settings and probes
        L.np_decode_set_staging.argtypes = [i64, i32]
        for b, t in [(-1, 0), ((1 << 30) + 1, 0), (1 << 20, -1), (1 << 20, 65)]:
            assert L.np_decode_set_staging(b, t) == EINVAL, (b, t)
        L.np_probe_read.argtypes = [vp, i64, vp, vp]
        L.np_probe_copy.argtypes = [vp, vp, i64, vp]
        L.np_probe_read_set.argtypes = [vp, i32, i64, i32, vp, vp]
        assert L.np_probe_read(None, 16, x.ctypes.data, None) == EINVAL
        assert L.np_probe_read(x.ctypes.data, 15, x.ctypes.data, None) == EINVAL
        assert L.np_probe_copy(None, x.ctypes.data, 16, None) == EINVAL
        assert L.np_probe_copy(x.ctypes.data, x.ctypes.data, 17, None) == EINVAL
        ptrs = (ctypes.c_void_p * 1)(x.ctypes.data)
        assert L.np_probe_read_set(ptrs, 0, 16, 1, x.ctypes.data, None) == EINVAL
        assert L.np_probe_read_set(ptrs, 1, 16, 0, x.ctypes.data, None) == EINVAL
        assert L.np_probe_read_set(None, 1, 16, 1, x.ctypes.data, None) == EINVAL
        assert isinstance(L.np_last_error(), bytes)
        print("host checks ok")
    ''')
    out = _run([sys.executable, "-c", script, lib], _env({}))
    assert "host checks ok" in out
