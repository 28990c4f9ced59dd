"""Hashes and digests of concept lists, written for the tests.

Intent hash h chains the SplitMix64 output function f over the intent's 64-bit
words: h = f(...f(f(0 ^ w0) ^ w1)...).  Extent hash g sums f over the extent
bitmap's words, each keyed by its index: g = sum over k of f(a_k ^ f(k)).
digest = sum over intents of h(B) mod 2^64 (order-free); the positional
digests weight every hash by the row's position: sum over i of i * h_i.
f is the output function of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014;
constants of Vigna's public splitmix64.c).  Three implementations: plain Python
integers (the reference), numpy uint64 arrays, and torch int64 tensors (two's
complement wrap-around, logical shifts by masking) for device-resident
intents.  The oracle computes the same digest in C; nothing here is shared
with it or with the GPU library.
"""

import numpy as np

MASK = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB


def mix_py(z: int) -> int:
    z = (z + GOLDEN) & MASK
    z = ((z ^ (z >> 30)) * MUL1) & MASK
    z = ((z ^ (z >> 27)) * MUL2) & MASK
    return z ^ (z >> 31)


def digest_py(intents) -> int:
    total = 0
    for row in np.asarray(intents, dtype=np.uint64):
        h = 0
        for w in row:
            h = mix_py(h ^ int(w))
        total = (total + h) & MASK
    return total


def digest_np(intents: np.ndarray, chunk: int = 1 << 20) -> int:
    a = np.ascontiguousarray(intents, dtype=np.uint64)
    total = np.uint64(0)
    with np.errstate(over="ignore"):
        for s in range(0, a.shape[0], chunk):
            h = np.zeros(min(chunk, a.shape[0] - s), dtype=np.uint64)
            for k in range(a.shape[1]):
                z = (h ^ a[s:s + chunk, k]) + np.uint64(GOLDEN)
                z = (z ^ (z >> np.uint64(30))) * np.uint64(MUL1)
                z = (z ^ (z >> np.uint64(27))) * np.uint64(MUL2)
                h = z ^ (z >> np.uint64(31))
            total = total + h.sum(dtype=np.uint64)
    return int(total)


def _signed(x: int) -> int:
    return x - (1 << 64) if x >= 1 << 63 else x


def digest_torch(intents, chunk: int = 1 << 24) -> int:
    """intents: int64 tensor [K, W] (the uint64 words reinterpreted), any device."""
    import torch

    g, m1, m2 = _signed(GOLDEN), _signed(MUL1), _signed(MUL2)

    def shr(z, k):  # logical right shift of int64 as uint64
        return (z >> k) & ((1 << (64 - k)) - 1)

    total = 0
    for s in range(0, intents.shape[0], chunk):
        block = intents[s:s + chunk]
        h = torch.zeros(block.shape[0], dtype=torch.int64, device=block.device)
        for k in range(block.shape[1]):
            z = (h ^ block[:, k]) + g
            z = (z ^ shr(z, 30)) * m1
            z = (z ^ shr(z, 27)) * m2
            h = z ^ shr(z, 31)
        total = (total + int(h.sum())) & MASK
    return total


# --- per-row hashes and positional digests ---------------------------------------------

def extent_hash_py(words) -> int:
    """g of one bitmap row (plain Python integers)."""
    h = 0
    for k, w in enumerate(words):
        h = (h + mix_py(int(w) ^ mix_py(k))) & MASK
    return h


def intent_hashes_np(intents: np.ndarray) -> np.ndarray:
    """h of every row, uint64 [K]."""
    a = np.ascontiguousarray(intents, dtype=np.uint64)
    h = np.zeros(a.shape[0], dtype=np.uint64)
    with np.errstate(over="ignore"):
        for k in range(a.shape[1]):
            h = _mix_np(h ^ a[:, k])
    return h


def _mix_np(z):
    with np.errstate(over="ignore"):
        z = z + np.uint64(GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MUL1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MUL2)
        return z ^ (z >> np.uint64(31))


def extent_hashes_np(extents: np.ndarray, chunk: int = 1 << 14) -> np.ndarray:
    """g of every row, uint64 [K]."""
    a = np.ascontiguousarray(extents, dtype=np.uint64)
    keys = _mix_np(np.arange(a.shape[1], dtype=np.uint64))
    out = np.zeros(a.shape[0], dtype=np.uint64)
    with np.errstate(over="ignore"):
        for s in range(0, a.shape[0], chunk):
            out[s:s + chunk] = _mix_np(a[s:s + chunk] ^ keys[None, :]).sum(axis=1, dtype=np.uint64)
    return out


def positional_py(hashes, start: int = 0) -> int:
    """sum over i of (start + i) * hashes[i], mod 2^64."""
    total = 0
    for i, h in enumerate(hashes):
        total = (total + (start + i) * int(h)) & MASK
    return total


def positional_np(hashes: np.ndarray, start: int = 0) -> int:
    h = np.asarray(hashes, dtype=np.uint64)
    with np.errstate(over="ignore"):
        pos = np.arange(start, start + h.shape[0], dtype=np.uint64)
        return int((pos * h).sum(dtype=np.uint64))


def _mix_torch(z):
    g, m1, m2 = _signed(GOLDEN), _signed(MUL1), _signed(MUL2)

    def shr(v, k):  # logical right shift of int64 as uint64
        return (v >> k) & ((1 << (64 - k)) - 1)

    z = z + g
    z = (z ^ shr(z, 30)) * m1
    z = (z ^ shr(z, 27)) * m2
    return z ^ shr(z, 31)


def intent_hashes_torch(intents):
    """h of every row of an int64 tensor [K, W] (any device), as int64 [K]."""
    import torch

    h = torch.zeros(intents.shape[0], dtype=torch.int64, device=intents.device)
    for k in range(intents.shape[1]):
        h = _mix_torch(h ^ intents[:, k])
    return h


def extent_hashes_torch(extents, chunk: int = 0):
    """g of every row of an int64 tensor [K, W] (any device), as int64 [K]."""
    import torch

    w = extents.shape[1]
    if chunk <= 0:
        chunk = max(1, (1 << 27) // w)  # about 1 GB per temporary
    keys = _mix_torch(torch.arange(w, dtype=torch.int64, device=extents.device))
    out = torch.empty(extents.shape[0], dtype=torch.int64, device=extents.device)
    for s in range(0, extents.shape[0], chunk):
        out[s:s + chunk] = _mix_torch(extents[s:s + chunk] ^ keys[None, :]).sum(dim=1)
    return out


def positional_torch(hashes, start: int = 0) -> int:
    """sum over i of (start + i) * hashes[i] mod 2^64 for an int64 tensor."""
    import torch

    pos = torch.arange(hashes.shape[0], dtype=torch.int64, device=hashes.device) + start
    return int((pos * hashes).sum()) & MASK


def to_u64(x: int) -> int:
    return x & MASK
