"""CPU oracle for formal-concept enumeration.

TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library imports, links or runs
anything in this package; only the tests, the smoke check and the CPU-baseline
leg of the benchmark do.  It shares no code with the GPU path.

* :func:`cbo` runs the serial Close-by-One in ``cbo.c`` (built with gcc into
  ``liboracle_cbo.so`` next to it) and returns sorted intents, extents and the
  work counters.
* :func:`cbo_digest` runs the same search from ``cbo_digest.c`` with object
  lists and no concept store, returning the counters, an order-independent
  digest of the intents and positional digests of intents and extents (every
  concept weighted by its output position), also per subtree of the root's
  children (for contexts whose concepts do not fit in memory).
* :func:`cover_edges` lists the lattice's cover edges (``cover.c``): the lower
  covers of every concept of a sorted concept list, as output positions.
* :func:`model_bytes` evaluates the algorithmic byte count of an enumeration
  (the formula documented with ``fcbo_stats`` in the library header) from the
  oracle's counters.
* :mod:`oracle.brute` holds two brute-force enumerations written straight from
  the definition of a concept, plus the CbO generation tree derived from the
  closed sets alone; they pin the C oracle on small contexts.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cbo.c")
_SRC_DIGEST = os.path.join(_HERE, "cbo_digest.c")
_SRC_COVER = os.path.join(_HERE, "cover.c")
_LIB = os.path.join(_HERE, "liboracle_cbo.so")


class _Result(ctypes.Structure):
    _fields_ = [
        ("n_concepts", ctypes.c_int64),
        ("tests", ctypes.c_int64),
        ("pairs", ctypes.c_int64),
        ("sum_nzw", ctypes.c_int64),
        ("sum_c", ctypes.c_int64),
        ("saturation_violations", ctypes.c_int64),
        ("sum_rl_objs", ctypes.c_int64),
        ("col_parents", ctypes.c_int64),
        ("col_nzw", ctypes.c_int64),
        ("col_child_objs", ctypes.c_int64),
        ("n_levels", ctypes.c_int32),
        ("truncated", ctypes.c_int32),
        ("level_concepts", ctypes.POINTER(ctypes.c_int64)),
        ("level_tests", ctypes.POINTER(ctypes.c_int64)),
        ("intents", ctypes.POINTER(ctypes.c_uint64)),
        ("extents", ctypes.POINTER(ctypes.c_uint64)),
        ("extent_hashes", ctypes.POINTER(ctypes.c_uint64)),
        ("wn", ctypes.c_int64),
        ("wm", ctypes.c_int64),
        ("seconds_enum", ctypes.c_double),
        ("seconds_sort", ctypes.c_double),
    ]


class _Subtree(ctypes.Structure):
    _fields_ = [
        ("size", ctypes.c_int64),
        ("hi0", ctypes.c_uint64),
        ("hi1", ctypes.c_uint64),
        ("he0", ctypes.c_uint64),
        ("he1", ctypes.c_uint64),
    ]


class _Digest(ctypes.Structure):
    _fields_ = [
        ("n_concepts", ctypes.c_int64),
        ("tests", ctypes.c_int64),
        ("pairs", ctypes.c_int64),
        ("sum_c", ctypes.c_int64),
        ("n_levels", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("level_concepts", ctypes.POINTER(ctypes.c_int64)),
        ("level_tests", ctypes.POINTER(ctypes.c_int64)),
        ("digest", ctypes.c_uint64),
        ("subtree_size", ctypes.c_int64),
        ("intent_digest", ctypes.c_uint64),
        ("intent_positional", ctypes.c_uint64),
        ("extent_digest", ctypes.c_uint64),
        ("extent_positional", ctypes.c_uint64),
        ("n_root_children", ctypes.c_int32),
        ("root_child_attr", ctypes.POINTER(ctypes.c_int32)),
        ("root_child", ctypes.POINTER(_Subtree)),
        ("seconds", ctypes.c_double),
    ]


def build(force: bool = False) -> str:
    """Compile ``cbo.c`` and ``cbo_digest.c`` into ``liboracle_cbo.so`` (plain gcc, -O2, no SIMD flags)."""
    srcs = [_SRC, _SRC_DIGEST, _SRC_COVER]
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        [os.path.getmtime(x) for x in srcs] + [os.path.getmtime(os.path.join(_HERE, "oracle_cbo.h"))]
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-D_POSIX_C_SOURCE=199309L", "-fPIC", "-shared", "-pthread",
             "-Wall", "-Wextra", "-o", tmp] + srcs,
            cwd=_HERE,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.oracle_cbo.argtypes = [
            ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(_Result),
        ]
        lib.oracle_cbo.restype = ctypes.c_int
        lib.oracle_free.argtypes = [ctypes.POINTER(_Result)]
        lib.oracle_free.restype = None
        lib.oracle_cbo_digest.argtypes = [
            ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.POINTER(_Digest),
        ]
        lib.oracle_cbo_digest.restype = ctypes.c_int
        lib.oracle_digest_free.argtypes = [ctypes.POINTER(_Digest)]
        lib.oracle_digest_free.restype = None
        lib.oracle_cover_edges.argtypes = [
            ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
            ctypes.POINTER(ctypes.POINTER(ctypes.c_int64)), ctypes.POINTER(ctypes.c_int64),
        ]
        lib.oracle_cover_edges.restype = ctypes.c_int
        lib.oracle_cover_free.argtypes = [ctypes.POINTER(ctypes.c_int64)]
        lib.oracle_cover_free.restype = None
        _lib = lib
    return _lib


@dataclass
class OracleResult:
    n_objects: int
    n_attrs: int
    n_concepts: int
    tests: int
    pairs: int
    sum_nzw: int
    sum_c: int
    saturation_violations: int
    rowlocal_max: int
    sum_rl_objs: int
    col_parents: int
    col_nzw: int
    col_child_objs: int
    n_levels: int
    truncated: bool
    level_concepts: np.ndarray  # int64 [n_levels]
    level_tests: np.ndarray     # int64 [n_levels]
    intents: np.ndarray         # uint64 [K, wm], lexicographic over attributes 0..M-1
    extents: np.ndarray | None  # uint64 [K, wn] in the same order
    extent_hashes: np.ndarray | None  # uint64 [K] g(extent) in the same order
    seconds_enum: float
    seconds_sort: float

    @property
    def wn(self) -> int:
        return (self.n_objects + 63) // 64

    @property
    def wm(self) -> int:
        return (self.n_attrs + 63) // 64


KEEP_EXTENTS = 1
HASH_EXTENTS = 2


def rowlocal_threshold(n_attrs: int) -> int:
    """T of the byte model: parents with at most T objects count as row-local (the
    rule stated with fcbo_stats: 4096 objects up to 512 attributes, else 64)."""
    return 4096 if (n_attrs + 63) // 64 <= 8 else 64


def cbo(rows: np.ndarray, n_attrs: int, keep_extents: bool = True, max_tests: int = -1,
        hash_extents: bool = False, rowlocal_max: int | None = None) -> OracleResult:
    """Run the serial CbO oracle on packed rows (uint64 [N, ceil(M/64)])."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.uint64)
    if rows.ndim != 2:
        raise ValueError("rows must be 2-D")
    n = rows.shape[0]
    if rowlocal_max is None:
        rowlocal_max = rowlocal_threshold(n_attrs)
    res = _Result()
    flags = (KEEP_EXTENTS if keep_extents else 0) | (HASH_EXTENTS if hash_extents else 0)
    rc = lib.oracle_cbo(
        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n, int(n_attrs), rows.shape[1],
        flags, int(max_tests), int(rowlocal_max), ctypes.byref(res),
    )
    if rc != 0:
        raise RuntimeError("oracle_cbo failed with %d" % rc)
    try:
        k, wn, wm = res.n_concepts, res.wn, res.wm
        nl = res.n_levels
        intents = np.ctypeslib.as_array(res.intents, shape=(k * wm,)).reshape(k, wm).copy()
        extents = None
        if keep_extents:
            extents = np.ctypeslib.as_array(res.extents, shape=(k * wn,)).reshape(k, wn).copy()
        ehash = None
        if hash_extents:
            ehash = np.ctypeslib.as_array(res.extent_hashes, shape=(k,)).copy()
        lc = np.ctypeslib.as_array(res.level_concepts, shape=(nl,)).copy()
        lt = np.ctypeslib.as_array(res.level_tests, shape=(nl,)).copy()
        return OracleResult(
            n_objects=n, n_attrs=int(n_attrs), n_concepts=k, tests=res.tests, pairs=res.pairs,
            sum_nzw=res.sum_nzw, sum_c=res.sum_c,
            saturation_violations=res.saturation_violations, rowlocal_max=int(rowlocal_max),
            sum_rl_objs=res.sum_rl_objs, col_parents=res.col_parents, col_nzw=res.col_nzw,
            col_child_objs=res.col_child_objs, n_levels=nl,
            truncated=bool(res.truncated), level_concepts=lc, level_tests=lt,
            intents=intents, extents=extents, extent_hashes=ehash, seconds_enum=res.seconds_enum,
            seconds_sort=res.seconds_sort,
        )
    finally:
        lib.oracle_free(ctypes.byref(res))


@dataclass
class DigestResult:
    n_concepts: int
    tests: int
    pairs: int
    sum_c: int
    n_levels: int
    level_concepts: np.ndarray  # int64 [n_levels]
    level_tests: np.ndarray     # int64 [n_levels]
    digest: int                 # sum of the SplitMix64 chains of the intents, mod 2^64
    intent_digest: int          # the same sum, from the subtree summaries
    intent_positional: int      # sum over output positions i of i * h(intent_i), mod 2^64
    extent_digest: int          # sum of the extent hashes g, mod 2^64
    extent_positional: int      # sum over i of i * g(extent_i), mod 2^64
    subtree_size: int
    root_children: list         # per child of the root, output order: dict(attr, size, hi0, hi1, he0, he1)
    threads: int
    seconds: float


def cbo_digest(rows: np.ndarray, n_attrs: int, threads: int = 1) -> DigestResult:
    """Counters and intent digest of the CbO search, with no concept store."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.uint64)
    if rows.ndim != 2:
        raise ValueError("rows must be 2-D")
    res = _Digest()
    rc = lib.oracle_cbo_digest(
        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), rows.shape[0], int(n_attrs), rows.shape[1],
        int(threads), ctypes.byref(res),
    )
    if rc != 0:
        raise RuntimeError("oracle_cbo_digest failed with %d" % rc)
    try:
        nl = res.n_levels
        kids = []
        for i in range(res.n_root_children):
            t = res.root_child[i]
            kids.append({"attr": int(res.root_child_attr[i]), "size": int(t.size), "hi0": int(t.hi0),
                         "hi1": int(t.hi1), "he0": int(t.he0), "he1": int(t.he1)})
        return DigestResult(
            n_concepts=res.n_concepts, tests=res.tests, pairs=res.pairs, sum_c=res.sum_c, n_levels=nl,
            level_concepts=np.ctypeslib.as_array(res.level_concepts, shape=(nl,)).copy(),
            level_tests=np.ctypeslib.as_array(res.level_tests, shape=(nl,)).copy(),
            digest=int(res.digest), intent_digest=int(res.intent_digest),
            intent_positional=int(res.intent_positional), extent_digest=int(res.extent_digest),
            extent_positional=int(res.extent_positional), subtree_size=int(res.subtree_size),
            root_children=kids, threads=res.threads, seconds=res.seconds,
        )
    finally:
        lib.oracle_digest_free(ctypes.byref(res))


def model_bytes(r: OracleResult) -> int:
    """Algorithmic bytes of the enumeration (the formula stated with fcbo_stats):
    every concept read once as a parent (intent, cursor, list bounds); the list
    entry and row of every object of a row-local parent (|A| <= T); for every
    larger parent its extent bitmap, the column words at its extent's non-zero
    words per test and the rows of its children's objects; every child written
    (intent, cursor, list offset, list); the root's rows and list."""
    wn = (r.n_objects + 63) // 64
    wm = (r.n_attrs + 63) // 64
    k = r.n_concepts
    b = k * (8 * wm + 4 + 16)
    b += r.sum_rl_objs * (4 + 8 * wm)
    b += r.col_parents * 8 * wn
    b += r.col_nzw * 8
    b += r.col_child_objs * 8 * wm
    b += (k - 1) * (8 * wm + 4 + 8) + 4 * r.sum_c
    b += r.n_objects * (8 * wm + 4)
    return b


def cover_edges(rows: np.ndarray, n_attrs: int, intents: np.ndarray):
    """Lower covers of every concept of a complete, sorted concept list.

    Returns (offsets int64 [K + 1], targets int64 [E]): the lower covers of the
    concept at position i are targets[offsets[i]:offsets[i + 1]], ascending."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.uint64)
    intents = np.ascontiguousarray(intents, dtype=np.uint64)
    k = intents.shape[0]
    offsets = np.zeros(k + 1, dtype=np.int64)
    tg = ctypes.POINTER(ctypes.c_int64)()
    ne = ctypes.c_int64(0)
    rc = lib.oracle_cover_edges(
        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), rows.shape[0], int(n_attrs), rows.shape[1],
        intents.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), k,
        offsets.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(tg), ctypes.byref(ne),
    )
    if rc != 0:
        raise RuntimeError("oracle_cover_edges failed with %d" % rc)
    try:
        targets = np.ctypeslib.as_array(tg, shape=(ne.value,)).copy() if ne.value else np.zeros(0, np.int64)
    finally:
        lib.oracle_cover_free(tg)
    return offsets, targets
