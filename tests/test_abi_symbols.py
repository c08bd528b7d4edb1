"""The C-ABI library loads (no GPU needed) and exports every function include/np.h declares."""
import ctypes
import os
import re

from delta_prefetched_ffn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "np.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(np_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["np_layer_create", "np_delta_assign", "np_scatter_rows", "np_sparse_ffn",
                     "np_decode_step"]:
        assert required in names
    assert sorted(binding.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_last_error_is_empty_string_initially_and_null_args_fail_on_host():
    lib = binding.lib()
    assert isinstance(lib.np_last_error(), bytes)
    # host-side validation runs before any device call: NULL desc -> NP_EINVAL
    assert lib.np_layer_create(None, None) == binding.NP_EINVAL
    assert b"NULL" in lib.np_last_error()
    assert lib.np_delta_assign(None, 0, 0, None) == binding.NP_EINVAL
    assert lib.np_scatter_rows(None, None) == binding.NP_EINVAL
    assert lib.np_sparse_ffn(None, None, None, None) == binding.NP_EINVAL
    assert lib.np_decode_step(None, 0, None, None, None, None, None) == binding.NP_EINVAL
