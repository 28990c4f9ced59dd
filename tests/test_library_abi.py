"""The C-ABI library builds, loads and exports every function of include/fcbo.h.

CPU only: no call here touches a device.
"""

import ctypes
import os
import re

import pytest

import closed_set_enumeration_amd as fca
from closed_set_enumeration_amd import build as fbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fcbo.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|void|const char \*)\s*(fcbo_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    fbuild.build(force=False)
    return ctypes.CDLL(fbuild.LIB)


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("fcbo_context_create", "fcbo_enumerate", "fcbo_destroy"):
        assert n in names
    assert set(names) == set(fca.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_error_strings(lib):
    assert fca.fcbo_error_string(fca.FCBO_OK) == "ok"
    assert "capacity" in fca.fcbo_error_string(fca.FCBO_ERR_CAPACITY)
    assert fca.fcbo_error_string(12345) == "unknown error"


def test_stats_struct_matches_header():
    # 14 u64 counters, 4 doubles, then per kernel class one double and one u64
    n = len(fca.KERNEL_CLASSES)
    assert ctypes.sizeof(fca.FcboStats) == 14 * 8 + 4 * 8 + n * 8 + n * 8
    text = open(HEADER).read()
    assert "FCBO_K_NUM_CLASSES = %d" % len(fca.KERNEL_CLASSES) in text


def test_null_arguments_are_rejected_without_a_device(lib):
    out = ctypes.c_void_p(123)
    lib.fcbo_context_create.restype = ctypes.c_int
    lib.fcbo_context_create.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_uint32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    # argument checks come before any HIP call
    assert lib.fcbo_context_create(None, 10, 10, 1, 0, None, ctypes.byref(out)) == fca.FCBO_ERR_INVALID_ARGUMENT
    assert out.value is None
    lib.fcbo_enumerate.restype = ctypes.c_int
    assert lib.fcbo_enumerate(None, None, None, 0, 0, None, None) == fca.FCBO_ERR_INVALID_ARGUMENT
    lib.fcbo_destroy(None)
