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


def header_stats_fields():
    """(name, type, count) of every field of fcbo_stats as the header declares it."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} fcbo_stats;", text, flags=re.S).group(1)
    consts = {"FCBO_K_NUM_CLASSES": int(re.search(r"FCBO_K_NUM_CLASSES = (\d+)", text).group(1))}
    out = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        m = re.fullmatch(r"(uint64_t|double)\s+(\w+)(?:\[(\w+)\])?", decl)
        assert m, decl
        out.append((m.group(2), m.group(1), consts[m.group(3)] if m.group(3) else 1))
    return out


def test_stats_struct_matches_header():
    ctype = {"uint64_t": ctypes.c_uint64, "double": ctypes.c_double}
    want = header_stats_fields()
    got = []
    for name, t in fca.FcboStats._fields_:
        if issubclass(t, ctypes.Array):
            got.append((name, t._type_, t._length_))
        else:
            got.append((name, t, 1))
    assert [(n, ctype[t], c) for n, t, c in want] == got
    assert len(fca.KERNEL_CLASSES) == dict((n, c) for n, _, c in want)["kernel_ms"]
    # the measurement record comes first, as the header documents
    assert [n for n, _, _ in want[:8]] == ["n_concepts", "closure_tests", "item_pairs", "n_levels", "enumerate_ms",
                                          "closure_kernel_ms", "sort_ms", "model_bytes"]


def test_error_codes_match_header():
    text = open(HEADER).read()
    for name in ("FCBO_OK", "FCBO_ERR_INVALID_ARGUMENT", "FCBO_ERR_OUT_OF_MEMORY", "FCBO_ERR_DEVICE",
                 "FCBO_ERR_CAPACITY", "FCBO_ERR_LIMIT", "FCBO_ERR_SCRATCH"):
        v = int(re.search(r"\b%s = (-?\d+)" % name, text).group(1))
        assert getattr(fca, name) == v, name
    assert "32-bit" in fca.fcbo_error_string(fca.FCBO_ERR_LIMIT)
    assert "static scratch" in fca.fcbo_error_string(fca.FCBO_ERR_SCRATCH)
    assert "(64u << 20)" in text and fca.FCBO_STATIC_SCRATCH_BYTES == 64 << 20


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
    lib.fcbo_enumerate_bounded.restype = ctypes.c_int
    assert lib.fcbo_enumerate_bounded(None, None, None, ctypes.c_uint64(1), None, None, 0, None,
                                      None) == fca.FCBO_ERR_INVALID_ARGUMENT
    lib.fcbo_write_range.restype = ctypes.c_int
    assert lib.fcbo_write_range(None, ctypes.c_uint64(0), ctypes.c_uint64(0), None, None) == fca.FCBO_ERR_INVALID_ARGUMENT
    lib.fcbo_set_memory_limit.restype = ctypes.c_int
    assert lib.fcbo_set_memory_limit(None, ctypes.c_uint64(1)) == fca.FCBO_ERR_INVALID_ARGUMENT
    lib.fcbo_enumerate_static.restype = ctypes.c_int
    assert lib.fcbo_enumerate_static(None, ctypes.c_int64(10), ctypes.c_int64(10), ctypes.c_int64(1), 0, None,
                                     None, None, ctypes.c_uint64(0), None, None) == fca.FCBO_ERR_INVALID_ARGUMENT
    # a context whose rows and columns alone take more than half the scratch is
    # refused before any device call (4,000,000 x 64: 32 MB of rows, 32 MB of columns)
    assert lib.fcbo_enumerate_static(ctypes.c_void_p(8), ctypes.c_int64(4_000_000), ctypes.c_int64(64),
                                     ctypes.c_int64(1), 1, None, None, None, ctypes.c_uint64(0), None,
                                     None) == fca.FCBO_ERR_SCRATCH
    lib.fcbo_destroy(None)
