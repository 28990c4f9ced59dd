"""Formal-concept enumeration on MI355X: Python binding of libfcbo.so.

The functions named like the C ABI (``fcbo_context_create``, ``fcbo_enumerate``,
``fcbo_enumerate_bounded``, ``fcbo_write_range``, ``fcbo_set_memory_limit``,
``fcbo_level_counts``, ``fcbo_copy_columns``, ``fcbo_destroy``,
``fcbo_error_string``, ...) only marshal arguments; every step of the enumeration
runs in the HIP kernels of the library.  :class:`Context` is a convenience
wrapper that takes device buffers and the stream from PyTorch.

There is no CPU fallback: if ``libfcbo.so`` has not been built, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfcbo.so")

FCBO_OK = 0
FCBO_ERR_INVALID_ARGUMENT = -1
FCBO_ERR_OUT_OF_MEMORY = -2
FCBO_ERR_DEVICE = -3
FCBO_ERR_CAPACITY = -4
FCBO_ERR_LIMIT = -5
FCBO_ERR_SCRATCH = -6
FCBO_ERR_STOPPED = -7
FCBO_STATIC_SCRATCH_BYTES = 64 << 20

FCBO_ROWS_ON_DEVICE = 1
FCBO_TINY_BUFFERS = 2
FCBO_REUSE_RESULT = 1
FCBO_PROFILE = 2
FCBO_ONE_SUBTREE_PER_BATCH = 4
FCBO_TASK_POOL = 16
FCBO_SPLIT_ROOT_CHILDREN = 8

KERNEL_CLASSES = ("count", "test_local", "test_medium", "test_big", "scan", "write_local", "write_medium",
                  "write_big", "order", "output")

EXPORTED = (
    "fcbo_context_create",
    "fcbo_enumerate",
    "fcbo_enumerate_bounded",
    "fcbo_write_range",
    "fcbo_copy_to_host",
    "fcbo_cover_edges",
    "fcbo_set_memory_limit",
    "fcbo_enumerate_static",
    "fcbo_level_counts",
    "fcbo_copy_columns",
    "fcbo_destroy",
    "fcbo_error_string",
)


class FcboStats(ctypes.Structure):
    _fields_ = [
        ("n_concepts", ctypes.c_uint64),
        ("closure_tests", ctypes.c_uint64),
        ("item_pairs", ctypes.c_uint64),
        ("n_levels", ctypes.c_uint64),
        ("enumerate_ms", ctypes.c_double),
        ("closure_kernel_ms", ctypes.c_double),
        ("sort_ms", ctypes.c_double),
        ("model_bytes", ctypes.c_uint64),
        ("output_ms", ctypes.c_double),
        ("sum_child_objects", ctypes.c_uint64),
        ("output_bytes", ctypes.c_uint64),
        ("local_parents", ctypes.c_uint64),
        ("local_parent_objects", ctypes.c_uint64),
        ("medium_parents", ctypes.c_uint64),
        ("medium_parent_objects", ctypes.c_uint64),
        ("big_parents", ctypes.c_uint64),
        ("big_tests", ctypes.c_uint64),
        ("big_scanned_objects", ctypes.c_uint64),
        ("big_nonzero_words", ctypes.c_uint64),
        ("big_child_objects", ctypes.c_uint64),
        ("order_launches", ctypes.c_uint64),
        ("kernel_ms", ctypes.c_double * len(KERNEL_CLASSES)),
        ("kernel_launches", ctypes.c_uint64 * len(KERNEL_CLASSES)),
        ("batches", ctypes.c_uint64),
        ("batch_retries", ctypes.c_uint64),
        ("batch_splits", ctypes.c_uint64),
        ("peak_device_bytes", ctypes.c_uint64),
        ("level_redos", ctypes.c_uint64),
    ]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_ if name not in ("kernel_ms", "kernel_launches")}
        d["kernel_ms"] = dict(zip(KERNEL_CLASSES, list(self.kernel_ms)))
        d["kernel_launches"] = dict(zip(KERNEL_CLASSES, [int(x) for x in self.kernel_launches]))
        return d


class FcboError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__("%s failed: %s (%d)" % (what, fcbo_error_string(code), code))
        self.code = code


# int sink(void *user, uint64_t first, uint64_t count, const uint64_t *intents, const uint64_t *extents)
SINK_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                           ctypes.c_void_p)

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfcbo.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libfcbo.so not found at %s; build it with closed_set_enumeration_amd.build.build() "
            "(the enumeration has no CPU fallback)" % path
        )
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.fcbo_context_create.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
        P(ctypes.c_void_p),
    ]
    lib.fcbo_context_create.restype = ctypes.c_int
    lib.fcbo_enumerate.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, P(ctypes.c_uint64),
        P(FcboStats),
    ]
    lib.fcbo_enumerate.restype = ctypes.c_int
    lib.fcbo_enumerate_bounded.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_uint32, P(ctypes.c_uint64), P(FcboStats),
    ]
    lib.fcbo_enumerate_bounded.restype = ctypes.c_int
    lib.fcbo_write_range.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.fcbo_write_range.restype = ctypes.c_int
    lib.fcbo_copy_to_host.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_uint64, P(ctypes.c_double)]
    lib.fcbo_copy_to_host.restype = ctypes.c_int
    lib.fcbo_cover_edges.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                     P(ctypes.c_uint64), P(ctypes.c_double)]
    lib.fcbo_cover_edges.restype = ctypes.c_int
    lib.fcbo_set_memory_limit.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
    lib.fcbo_set_memory_limit.restype = ctypes.c_int
    lib.fcbo_enumerate_static.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, P(ctypes.c_uint64), P(FcboStats),
    ]
    lib.fcbo_enumerate_static.restype = ctypes.c_int
    lib.fcbo_level_counts.argtypes = [
        ctypes.c_void_p, P(ctypes.c_uint64), P(ctypes.c_uint64), ctypes.c_uint64, P(ctypes.c_uint64),
    ]
    lib.fcbo_level_counts.restype = ctypes.c_int
    lib.fcbo_copy_columns.argtypes = [ctypes.c_void_p, P(ctypes.c_uint64), ctypes.c_uint64]
    lib.fcbo_copy_columns.restype = ctypes.c_int
    lib.fcbo_destroy.argtypes = [ctypes.c_void_p]
    lib.fcbo_destroy.restype = None
    lib.fcbo_error_string.argtypes = [ctypes.c_int]
    lib.fcbo_error_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


# --- C-ABI-named wrappers ------------------------------------------------------

def fcbo_error_string(code: int) -> str:
    return load_library().fcbo_error_string(int(code)).decode()


def fcbo_context_create(rows_ptr: int, n_objects: int, n_attrs: int, row_stride_words: int, flags: int = 0,
                        hip_stream: int = 0) -> int:
    """Returns the context handle; raises FcboError on failure."""
    out = ctypes.c_void_p()
    rc = load_library().fcbo_context_create(
        ctypes.c_void_p(rows_ptr), n_objects, n_attrs, row_stride_words, flags, ctypes.c_void_p(hip_stream),
        ctypes.byref(out),
    )
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_context_create")
    return out.value


def fcbo_enumerate(ctx: int, intents_out_ptr: int, extents_out_ptr: int, capacity: int, flags: int = 0):
    """Returns (rc, n_concepts, FcboStats); FCBO_ERR_CAPACITY is returned, not raised."""
    k = ctypes.c_uint64(0)
    st = FcboStats()
    rc = load_library().fcbo_enumerate(
        ctypes.c_void_p(ctx), ctypes.c_void_p(intents_out_ptr or None), ctypes.c_void_p(extents_out_ptr or None),
        capacity, flags, ctypes.byref(k), ctypes.byref(st),
    )
    if rc not in (FCBO_OK, FCBO_ERR_CAPACITY):
        raise FcboError(rc, "fcbo_enumerate")
    return rc, k.value, st


def fcbo_enumerate_bounded(ctx: int, intents_buf_ptr: int, extents_buf_ptr: int, piece_rows: int, sink=None,
                           flags: int = 0):
    """Bounded-memory enumeration.  ``sink(first, count, intents_ptr, extents_ptr)`` is called
    once per piece with device pointers (0 for a buffer not given) and returns nothing to go
    on or a true value to stop.  Returns (n_concepts, FcboStats); raises FcboError on failure,
    or re-raises what the sink raised (the enumeration stops there)."""
    raised = []

    def trampoline(_user, first, count, ip, ep):
        try:
            return 1 if sink(first, count, ip or 0, ep or 0) else 0
        except BaseException as e:  # handed back to the caller after the C call returns
            raised.append(e)
            return 1

    cb = SINK_FN(trampoline) if sink is not None else None
    k = ctypes.c_uint64(0)
    st = FcboStats()
    rc = load_library().fcbo_enumerate_bounded(
        ctypes.c_void_p(ctx), ctypes.c_void_p(intents_buf_ptr or None), ctypes.c_void_p(extents_buf_ptr or None),
        piece_rows, ctypes.cast(cb, ctypes.c_void_p) if cb is not None else None, None, flags, ctypes.byref(k),
        ctypes.byref(st),
    )
    if raised:
        raise raised[0]
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_enumerate_bounded")
    return k.value, st


def fcbo_write_range(ctx: int, first: int, count: int, intents_out_ptr: int, extents_out_ptr: int) -> None:
    """Output rows [first, first + count) of the last enumeration; raises FcboError on failure."""
    rc = load_library().fcbo_write_range(ctypes.c_void_p(ctx), first, count, ctypes.c_void_p(intents_out_ptr or None),
                                         ctypes.c_void_p(extents_out_ptr or None))
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_write_range")


def fcbo_copy_to_host(ctx: int, first: int, count: int, host_intents_ptr: int, host_extents_ptr: int,
                      staging_rows: int) -> float:
    """Output rows [first, first + count) into host memory; returns the device ms."""
    ms = ctypes.c_double(0.0)
    rc = load_library().fcbo_copy_to_host(ctypes.c_void_p(ctx), first, count, ctypes.c_void_p(host_intents_ptr or None),
                                          ctypes.c_void_p(host_extents_ptr or None), staging_rows, ctypes.byref(ms))
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_copy_to_host")
    return ms.value


def fcbo_cover_edges(ctx: int, offsets_out_ptr: int, targets_out_ptr: int, capacity: int):
    """Returns (rc, n_edges, device ms); FCBO_ERR_CAPACITY is returned, not raised."""
    e = ctypes.c_uint64(0)
    ms = ctypes.c_double(0.0)
    rc = load_library().fcbo_cover_edges(ctypes.c_void_p(ctx), ctypes.c_void_p(offsets_out_ptr or None),
                                         ctypes.c_void_p(targets_out_ptr or None), capacity, ctypes.byref(e),
                                         ctypes.byref(ms))
    if rc not in (FCBO_OK, FCBO_ERR_CAPACITY):
        raise FcboError(rc, "fcbo_cover_edges")
    return rc, e.value, ms.value


def fcbo_set_memory_limit(ctx: int, nbytes: int) -> None:
    rc = load_library().fcbo_set_memory_limit(ctypes.c_void_p(ctx), int(nbytes))
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_set_memory_limit")


def fcbo_enumerate_static(rows_ptr: int, n_objects: int, n_attrs: int, row_stride_words: int, flags: int,
                          hip_stream: int, intents_out_ptr: int, extents_out_ptr: int, capacity: int):
    """The allocation-free call.  Returns (rc, n_concepts, FcboStats); FCBO_ERR_CAPACITY and
    FCBO_ERR_SCRATCH are returned, other errors raised."""
    k = ctypes.c_uint64(0)
    st = FcboStats()
    rc = load_library().fcbo_enumerate_static(
        ctypes.c_void_p(rows_ptr), n_objects, n_attrs, row_stride_words, flags, ctypes.c_void_p(hip_stream),
        ctypes.c_void_p(intents_out_ptr or None), ctypes.c_void_p(extents_out_ptr or None), capacity,
        ctypes.byref(k), ctypes.byref(st),
    )
    if rc not in (FCBO_OK, FCBO_ERR_CAPACITY, FCBO_ERR_SCRATCH):
        raise FcboError(rc, "fcbo_enumerate_static")
    return rc, k.value, st


def fcbo_level_counts(ctx: int):
    """(concepts per level, tests per level) of the last enumeration, as numpy uint64."""
    lib = load_library()
    nl = ctypes.c_uint64(0)
    rc = lib.fcbo_level_counts(ctypes.c_void_p(ctx), None, None, 0, ctypes.byref(nl))
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_level_counts")
    conc = np.zeros(nl.value, dtype=np.uint64)
    tests = np.zeros(nl.value, dtype=np.uint64)
    P = ctypes.POINTER(ctypes.c_uint64)
    rc = lib.fcbo_level_counts(ctypes.c_void_p(ctx), conc.ctypes.data_as(P), tests.ctypes.data_as(P), nl.value,
                               ctypes.byref(nl))
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_level_counts")
    return conc, tests


def fcbo_copy_columns(ctx: int, n_objects: int, n_attrs: int) -> np.ndarray:
    wn = (n_objects + 63) // 64
    out = np.zeros((n_attrs, wn), dtype=np.uint64)
    rc = load_library().fcbo_copy_columns(ctypes.c_void_p(ctx), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                          out.size)
    if rc != FCBO_OK:
        raise FcboError(rc, "fcbo_copy_columns")
    return out


def fcbo_destroy(ctx: int) -> None:
    if ctx:
        load_library().fcbo_destroy(ctypes.c_void_p(ctx))


# --- convenience wrapper over torch device buffers ----------------------------

@dataclass
class Result:
    n_concepts: int
    intents: "object"        # torch int64 tensor (K, wm) on the device, bits as in the C ABI
    extents: "object"        # torch int64 tensor (K, wn) or None
    stats: dict


class Context:
    """A formal context on the current HIP device.

    ``rows`` is a uint64 (N, ceil(M/64)) numpy array (copied from the host) or
    an int64/uint64 torch tensor already on the device.
    """

    def __init__(self, rows, n_attrs: int, stream=None, flags: int = 0):
        import torch

        if not torch.cuda.is_available():
            raise RuntimeError("no HIP device available")
        self._torch = torch
        self.n_attrs = int(n_attrs)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        extra = int(flags) & ~FCBO_ROWS_ON_DEVICE
        if isinstance(rows, np.ndarray):
            rows = np.ascontiguousarray(rows, dtype=np.uint64)
            if rows.ndim != 2:
                raise ValueError("rows must be 2-D")
            self.n_objects = rows.shape[0]
            ptr, stride, flags = rows.ctypes.data, rows.shape[1], 0
            keep = rows
        else:
            if rows.dim() != 2 or not rows.is_cuda:
                raise ValueError("a torch rows tensor must be 2-D and on the device")
            rows = rows.contiguous()
            self.n_objects = rows.shape[0]
            ptr, stride, flags = rows.data_ptr(), rows.shape[1], FCBO_ROWS_ON_DEVICE
            keep = rows
        self.wn = (self.n_objects + 63) // 64
        self.wm = (self.n_attrs + 63) // 64
        self.device = torch.cuda.current_device()
        self.handle = fcbo_context_create(ptr, self.n_objects, self.n_attrs, stride, flags | extra,
                                          self.stream.cuda_stream)
        del keep

    def close(self):
        if getattr(self, "handle", None):
            fcbo_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def count(self, pool: bool = False) -> int:
        """Enumerate (keeping the result in the context) and return K."""
        rc, k, _ = fcbo_enumerate(self.handle, 0, 0, 0, FCBO_TASK_POOL if pool else 0)
        if rc != FCBO_ERR_CAPACITY:  # a context has at least one concept, so no call with capacity 0 succeeds
            raise FcboError(rc, "fcbo_enumerate")
        return k

    def alloc_outputs(self, capacity: int, extents: bool = True):
        torch = self._torch
        dev = torch.device("cuda", torch.cuda.current_device())
        ints = torch.empty((max(capacity, 1), self.wm), dtype=torch.int64, device=dev)
        exts = torch.empty((max(capacity, 1), self.wn), dtype=torch.int64, device=dev) if extents else None
        return ints, exts

    def _check_buffer(self, t, width, what):
        """Shape, type, layout and device of a caller output buffer (before any launch)."""
        torch = self._torch
        if not isinstance(t, torch.Tensor):
            raise ValueError("%s must be a torch tensor" % what)
        if t.dim() != 2 or t.shape[1] != width:
            raise ValueError("%s must be 2-D with %d words per row, got %s" % (what, width, tuple(t.shape)))
        if t.element_size() != 8 or t.dtype.is_floating_point or t.dtype.is_complex:
            raise ValueError("%s must hold 64-bit integer words, got %s" % (what, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % what)
        if not t.is_cuda or t.device.index != self.device:
            raise ValueError("%s must be on the context's device cuda:%d" % (what, self.device))
        return t.shape[0]

    def enumerate_into(self, intents, extents, flags: int = 0):
        """One full call into preallocated buffers; returns (rc, K, stats dict)."""
        cap = self._check_buffer(intents, self.wm, "intents")
        if extents is not None:
            cap = min(cap, self._check_buffer(extents, self.wn, "extents"))
        rc, k, st = fcbo_enumerate(
            self.handle, intents.data_ptr(), extents.data_ptr() if extents is not None else 0, cap, flags
        )
        return rc, k, st.as_dict()

    def write_range(self, first: int, intents=None, extents=None):
        """Output rows [first, first + rows) of the last enumeration into the given buffers."""
        if intents is None and extents is None:
            raise ValueError("give an intent or an extent buffer")
        rows = None
        if intents is not None:
            rows = self._check_buffer(intents, self.wm, "intents")
        if extents is not None:
            r = self._check_buffer(extents, self.wn, "extents")
            if rows is not None and r != rows:
                raise ValueError("intent and extent buffers differ in rows")
            rows = r
        fcbo_write_range(self.handle, first, rows, intents.data_ptr() if intents is not None else 0,
                         extents.data_ptr() if extents is not None else 0)

    def cover_edges(self):
        """Lower covers of every concept of the last enumeration: (offsets int64 [K + 1],
        targets int32 [E]) on the device, in output positions, and the device ms of the
        counting and the writing call together."""
        torch = self._torch
        rc, e, ms_count = fcbo_cover_edges(self.handle, 0, 0, 0)
        if rc != FCBO_ERR_CAPACITY:
            raise FcboError(rc, "fcbo_cover_edges")
        dev = torch.device("cuda", self.device)
        k = fcbo_level_counts(self.handle)[0].sum()
        offsets = torch.empty(int(k) + 1, dtype=torch.int64, device=dev)
        targets = torch.empty(max(e, 1), dtype=torch.int32, device=dev)
        rc, e2, ms = fcbo_cover_edges(self.handle, offsets.data_ptr(), targets.data_ptr(), targets.shape[0])
        if rc != FCBO_OK or e2 != e:
            raise FcboError(rc, "fcbo_cover_edges")
        return offsets, targets[:e], ms_count + ms

    def copy_to_host(self, first: int, count: int, intents=None, extents=None, staging_rows: int = 1 << 20):
        """Output rows [first, first + count) into host arrays (numpy uint64 or CPU torch
        tensors, C-contiguous, count x W words); returns the device ms."""
        def ptr(a, width, what):
            if a is None:
                return 0
            if isinstance(a, np.ndarray):
                ok = a.dtype == np.uint64 and a.flags["C_CONTIGUOUS"] and a.ndim == 2
                p = a.ctypes.data
            else:
                ok = (not a.is_cuda) and a.element_size() == 8 and a.is_contiguous() and a.dim() == 2
                p = a.data_ptr()
            if not ok or a.shape[0] < count or a.shape[1] != width:
                raise ValueError("%s must be a C-contiguous host array of at least %d x %d 64-bit words"
                                 % (what, count, width))
            return p
        if intents is None and extents is None:
            raise ValueError("give an intent or an extent array")
        return fcbo_copy_to_host(self.handle, first, count, ptr(intents, self.wm, "intents"),
                                 ptr(extents, self.wn, "extents"), staging_rows)

    def enumerate_bounded(self, sink=None, piece_rows: int = 1 << 20, intents: bool = True, extents: bool = True,
                          profile: bool = False, flags: int = 0):
        """Enumerate in bounded device memory (cap it with set_memory_limit): ``sink(first,
        intents, extents)`` gets each piece as device tensors of ``count`` rows (views of
        the piece buffers, valid only during the call; None for an output not asked for)
        at output positions [first, first + count).  Returns (K, stats dict)."""
        torch = self._torch
        dev = torch.device("cuda", self.device)
        rows = max(1, int(piece_rows))
        ib = torch.empty((rows, self.wm), dtype=torch.int64, device=dev) if intents else None
        eb = torch.empty((rows, self.wn), dtype=torch.int64, device=dev) if extents else None

        def piece(first, count, _ip, _ep):
            return sink(first, ib[:count] if ib is not None else None, eb[:count] if eb is not None else None)

        k, st = fcbo_enumerate_bounded(self.handle, ib.data_ptr() if ib is not None else 0,
                                       eb.data_ptr() if eb is not None else 0, rows,
                                       piece if sink is not None else None,
                                       flags | (FCBO_PROFILE if profile else 0))
        return k, st.as_dict()

    def set_memory_limit(self, nbytes: int) -> None:
        fcbo_set_memory_limit(self.handle, nbytes)

    def enumerate(self, extents: bool = True, profile: bool = False, pool: bool = False) -> Result:
        k = self.count(pool)
        ints, exts = self.alloc_outputs(k, extents)
        flags = FCBO_REUSE_RESULT | (FCBO_PROFILE if profile else 0)
        rc, k2, st = self.enumerate_into(ints, exts, flags)
        if rc != FCBO_OK or k2 != k:
            raise FcboError(rc, "fcbo_enumerate")
        return Result(k, ints[:k], exts[:k] if exts is not None else None, st)

    def level_counts(self):
        return fcbo_level_counts(self.handle)

    def columns(self) -> np.ndarray:
        return fcbo_copy_columns(self.handle, self.n_objects, self.n_attrs)
