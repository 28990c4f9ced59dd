"""Seeded 0/1 formal contexts and their LSB-first uint64 row packing.

A formal context is a boolean matrix ``cells[g, m]`` (object g has attribute m).
Rows are packed LSB-first into 64-bit words: attribute m of object g is bit
``m & 63`` of word ``m >> 6`` of row g; bits past the last attribute are zero.

The five named workloads follow fixed recipes, every draw taken from
``numpy.random.default_rng(seed)`` in the order written below, so the same
seed always gives the same bytes.
"""

from __future__ import annotations

import hashlib

import numpy as np

GENERATOR_VERSION = "synth-contexts-1"


def words(n_bits: int) -> int:
    """Number of 64-bit words that hold ``n_bits`` bits."""
    return (int(n_bits) + 63) // 64


def pack_rows(cells: np.ndarray) -> np.ndarray:
    """Pack a bool (N, M) matrix into uint64 (N, ceil(M/64)), LSB-first."""
    cells = np.asarray(cells, dtype=bool)
    if cells.ndim != 2:
        raise ValueError("cells must be 2-D")
    n, m = cells.shape
    wm = words(m)
    padded = np.zeros((n, wm * 64), dtype=bool)
    padded[:, :m] = cells
    by = np.packbits(padded, axis=1, bitorder="little")  # (n, wm*8) bytes
    return np.ascontiguousarray(by).view("<u8").reshape(n, wm).astype(np.uint64)


def unpack_rows(rows: np.ndarray, n_attrs: int) -> np.ndarray:
    """Inverse of :func:`pack_rows`."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.uint64))
    n = rows.shape[0]
    by = rows.view(np.uint8).reshape(n, -1)
    bits = np.unpackbits(by, axis=1, bitorder="little")
    return bits[:, :n_attrs].astype(bool)


def rows_sha256(rows: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(rows, dtype="<u8").tobytes()).hexdigest()


def _plant(rng, cells, count, n_obj, n_att):
    """Set ``count`` biclusters of n_obj random objects x n_att random attributes."""
    n, m = cells.shape
    for _ in range(count):
        objs = rng.choice(n, n_obj, replace=False)
        atts = rng.choice(m, n_att, replace=False)
        cells[np.ix_(objs, atts)] = True


def _zipf_capped_scale(exponent: float, n_ranks: int, target_mean: float, cap: float) -> float:
    """Scale c with mean_r min(c * r**-exponent, cap) == target_mean (bisection)."""
    r = np.arange(1, n_ranks + 1, dtype=np.float64)
    lo, hi = 0.0, 1.0
    while np.minimum(hi * r ** -exponent, cap).mean() < target_mean:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(mid * r ** -exponent, cap).mean() < target_mean:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _cfg_64x16():
    rng = np.random.default_rng(1)
    return rng.random((64, 16)) < 0.3


def _cfg_2000x64():
    rng = np.random.default_rng(2)
    p = np.full(64, 0.15)
    sat = rng.choice(64, 2, replace=False)
    p[sat] = 0.95
    return rng.random((2000, 64)) < p[None, :]


def _cfg_10000x128():
    rng = np.random.default_rng(3)
    ranks = rng.permutation(128) + 1  # rank of attribute a is ranks[a]
    p = 0.5 / ranks.astype(np.float64)  # Zipf s = 1.0, top column density 0.5
    cells = rng.random((10000, 128)) < p[None, :]
    _plant(rng, cells, 20, 200, 8)
    return cells


def _cfg_50000x400():
    rng = np.random.default_rng(4)
    m = 400
    dense = int(rng.integers(m))
    others = np.array([a for a in range(m) if a != dense])
    ranks = rng.permutation(m - 1) + 1
    c = _zipf_capped_scale(1.1, m - 1, 0.02, 0.5)
    p = np.empty(m)
    p[others] = np.minimum(c * ranks.astype(np.float64) ** -1.1, 0.5)
    p[dense] = 0.9
    cells = rng.random((50000, m)) < p[None, :]
    _plant(rng, cells, 40, 500, 6)
    return cells


def _cfg_20000x256():
    rng = np.random.default_rng(5)
    cells = rng.random((20000, 256)) < 0.1
    _plant(rng, cells, 50, 400, 10)
    return cells


# name -> (objects, attributes, builder)
CONFIGS = {
    "ctx64x16": (64, 16, _cfg_64x16),
    "ctx2000x64": (2000, 64, _cfg_2000x64),
    "ctx10000x128": (10000, 128, _cfg_10000x128),
    "ctx50000x400": (50000, 400, _cfg_50000x400),
    "ctx20000x256": (20000, 256, _cfg_20000x256),
}


def make_config(name: str, packed: bool = True):
    """Return the named workload: packed uint64 rows (default) or bool cells."""
    n, m, build = CONFIGS[name]
    cells = build()
    assert cells.shape == (n, m)
    return pack_rows(cells) if packed else cells


def random_context(seed: int, n: int, m: int, density: float) -> np.ndarray:
    """Small i.i.d. Bernoulli(density) context as a bool (n, m) matrix."""
    rng = np.random.default_rng(seed)
    return rng.random((n, m)) < density


# --- contexts with a structure known in closed form ---------------------------

def all_zero(n: int, m: int) -> np.ndarray:
    return np.zeros((n, m), dtype=bool)


def all_ones(n: int, m: int) -> np.ndarray:
    return np.ones((n, m), dtype=bool)


def diagonal(k: int) -> np.ndarray:
    """Object i has exactly attribute i."""
    return np.eye(k, dtype=bool)


def contranominal(k: int) -> np.ndarray:
    """Object i has every attribute except i."""
    return ~np.eye(k, dtype=bool)


def planted_bicluster(n: int, m: int, objs, atts) -> np.ndarray:
    cells = np.zeros((n, m), dtype=bool)
    cells[np.ix_(np.asarray(objs), np.asarray(atts))] = True
    return cells


def pad_with_full(cells: np.ndarray, extra_objects: int = 0, extra_attrs: int = 0) -> np.ndarray:
    """Append all-ones objects (rows) and all-ones attributes (columns)."""
    n, m = cells.shape
    out = np.ones((n + extra_objects, m + extra_attrs), dtype=bool)
    out[:n, :m] = cells
    return out
