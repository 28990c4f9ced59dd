"""Order-independent digest of a set of intents, written for the tests.

digest = sum over intents of h(B) mod 2^64, where h chains the SplitMix64
output function f over the intent's 64-bit words: h = f(...f(f(0 ^ w0) ^ w1)...).
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
