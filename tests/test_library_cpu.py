"""Host-side checks of the C-ABI library that need no GPU: it builds, loads,
and exports every function that include/gemv.h declares."""
import ctypes
import os
import re

import pytest

from memory_bound_gemv_row_amd import binding, build

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gemv_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if build.stale():
        build.build()
    return ctypes.CDLL(binding.LIB_PATH)


def test_header_declares_the_four_paths():
    names = _declared_functions()
    for n in ("gemv_f32", "gemv_f16", "gemv_f16x32", "gemv_f16_acc16", "gemv_q8", "gemv_q4", "gemv_status_string",
              "gemv_quantize_q8", "gemv_quantize_q4"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    binding.load()
    assert binding.status_string(0) == "ok"
    assert binding.status_string(1) == "invalid argument"
    assert binding.status_string(2).startswith("unsupported")
    assert binding.status_string(99) == "unknown status"


def test_gfx950_code_object_is_embedded():
    blob = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_torch_wrappers_reject_dimensions_beyond_int():
    # M and N cross the C ABI as int; a larger dimension must raise instead
    # of wrapping (2^32 + 16 would become 16)
    from types import SimpleNamespace

    from memory_bound_gemv_row_amd import binding

    big = SimpleNamespace(shape=((1 << 32) + 16, 4))
    for fn in (binding.gemv_f32, binding.gemv_f16, binding.gemv_f16x32, binding.gemv_f16_acc16):
        with pytest.raises(ValueError, match="int range"):
            fn(big, None)
    with pytest.raises(ValueError, match="int range"):
        binding.gemv_q8(big, None, None)
    with pytest.raises(ValueError, match="int range"):
        binding.gemv_q4(SimpleNamespace(shape=(4, 1 << 31)), None, None)
    with pytest.raises(ValueError, match="int range"):
        binding.softmax_f16(SimpleNamespace(shape=(1, 1 << 31)))
