"""Brute-force concept enumeration straight from the definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Sets are Python ints:
element e is bit e.  Everything here is slow on purpose and meant for small
contexts; it exists to pin the serial CbO oracle, not to be fast.

Definitions used (page "hnwysp.cn/news/97538", sections 1.1-1.2): X' of an
object set is the set of attributes every object of X has (all attributes for
the empty X); Y' of an attribute set is the set of objects having every
attribute of Y (all objects for the empty Y).  A concept is (A, B) with
A' = B and B' = A; intents are exactly the sets B with B'' = B.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


class Context:
    """A formal context as Python-int rows and columns."""

    def __init__(self, cells: np.ndarray):
        cells = np.asarray(cells, dtype=bool)
        self.n, self.m = cells.shape
        self.all_objects = (1 << self.n) - 1
        self.all_attrs = (1 << self.m) - 1
        self.rows = [sum(1 << int(a) for a in np.flatnonzero(cells[g])) for g in range(self.n)]
        self.cols = [sum(1 << int(g) for g in np.flatnonzero(cells[:, a])) for a in range(self.m)]

    def objects_of(self, attrs: int) -> int:
        """Y' : the objects that have every attribute in ``attrs``."""
        out = self.all_objects
        a = 0
        while attrs:
            if attrs & 1:
                out &= self.cols[a]
            attrs >>= 1
            a += 1
        return out

    def attrs_of(self, objs: int) -> int:
        """X' : the attributes that every object in ``objs`` has."""
        out = self.all_attrs
        g = 0
        while objs:
            if objs & 1:
                out &= self.rows[g]
            objs >>= 1
            g += 1
        return out

    def close(self, attrs: int) -> int:
        return self.attrs_of(self.objects_of(attrs))


def closed_intents_by_subsets(ctx: Context) -> set[int]:
    """Every S'' over all 2^M attribute subsets S (feasible for M <= ~16)."""
    return {ctx.close(s) for s in range(1 << ctx.m)}


def closed_intents_by_row_meets(ctx: Context) -> set[int]:
    """Intents as {M} plus every intersection of a non-empty set of object rows.

    B is an intent iff B = X' for some object set X; X' is the AND of the rows
    of X, and the empty X gives M.  The family is built by closing {M} under
    intersection with each row in turn.
    """
    fam = {ctx.all_attrs}
    for r in ctx.rows:
        fam |= {b & r for b in fam}
    return fam


def intent_key(b: int, m: int) -> str:
    """Sort key: the intent as its characteristic string over attributes 0..m-1."""
    return "".join("1" if (b >> e) & 1 else "0" for e in range(m))


def to_words(sets, nbits: int) -> np.ndarray:
    """Python-int sets -> uint64 [len, ceil(nbits/64)] in the given order."""
    wm = (nbits + 63) // 64
    out = np.zeros((len(sets), wm), dtype=np.uint64)
    mask = (1 << 64) - 1
    for i, s in enumerate(sets):
        for w in range(wm):
            out[i, w] = (s >> (64 * w)) & mask
    return out


def sorted_concepts(ctx: Context, intents: set[int]):
    """(intents uint64 [K, wm], extents uint64 [K, wn]) in lexicographic intent order."""
    order = sorted(intents, key=lambda b: intent_key(b, ctx.m))
    return to_words(order, ctx.m), to_words([ctx.objects_of(b) for b in order], ctx.n)


@dataclass
class TreeStats:
    """CbO generation-tree quantities derived from the closed sets alone."""

    n_concepts: int = 0
    tests: int = 0
    pairs: int = 0
    sum_nzw: int = 0
    sum_c: int = 0
    # the same sums split by a threshold T on the parent's extent size
    sum_rl_objs: int = 0      # objects of the parents with |A| <= T
    col_parents: int = 0      # parents with |A| > T
    col_nzw: int = 0          # sum over their tests of the non-zero words of A
    col_child_objs: int = 0   # objects of their children
    level_concepts: list = field(default_factory=list)
    level_tests: list = field(default_factory=list)
    parent: dict = field(default_factory=dict)  # intent -> parent intent (None for the top)
    cursor: dict = field(default_factory=dict)  # intent -> generating attribute (-1 for the top)


def _nonzero_words(x: int) -> int:
    c = 0
    while x:
        if x & ((1 << 64) - 1):
            c += 1
        x >>= 64
    return c


def cbo_tree(ctx: Context, intents: set[int], rowlocal_max: int = 1 << 62) -> TreeStats:
    """The Close-by-One tree over a complete set of intents, without searching.

    For a closed D other than the top intent T = {}'' let
        y(D) = the least m with (D n {0..m})'' = D.
    Then D is generated exactly once, from the parent (D n {0..y(D)-1})'' with
    attribute j = y(D), and its cursor is y(D); the top has cursor -1.  (Proof
    sketch: every node B with cursor y satisfies B = (B n {0..y})''; a child D
    of B at j has D n {0..j-1} = B n {0..j-1}, hence D = (D n {0..j})'' and
    B = (D n {0..j-1})'', and j is then forced to be the least such m.)
    From the cursors follow the closure tests (j > y, j not in B), the item
    pairs (j > y), the level of every concept and the byte-model sums, also
    split by the size of the parent's extent against ``rowlocal_max``.
    """
    top = ctx.close(0)
    cursor, parent = {}, {}
    for d in intents:
        if d == top:
            cursor[d], parent[d] = -1, None
            continue
        prefix = 0
        for m in range(ctx.m):
            prefix |= d & (1 << m)
            if ctx.close(prefix) == d:
                cursor[d] = m
                parent[d] = ctx.close(d & ((1 << m) - 1))
                break
        else:  # pragma: no cover - a closed set is reached by m = M-1 at the latest
            raise AssertionError("closed set never reached")
    level = {}

    def depth(d):
        path = []
        while d not in level:
            if parent[d] is None:
                level[d] = 0
                break
            path.append(d)
            d = parent[d]
        base = level[d]
        for i, x in enumerate(reversed(path)):
            level[x] = base + i + 1
        return level[path[0]] if path else base

    st = TreeStats(n_concepts=len(intents), parent=parent, cursor=cursor)
    for d in intents:
        depth(d)
    nlev = max(level.values()) + 1
    st.level_concepts = [0] * nlev
    st.level_tests = [0] * nlev
    for d in intents:
        lv = level[d]
        st.level_concepts[lv] += 1
        ext = ctx.objects_of(d)
        size = bin(ext).count("1")
        col = size > rowlocal_max
        if col:
            st.col_parents += 1
        else:
            st.sum_rl_objs += size
        y = cursor[d]
        for j in range(y + 1, ctx.m):
            st.pairs += 1
            if (d >> j) & 1:
                continue
            st.tests += 1
            st.level_tests[lv] += 1
            st.sum_nzw += _nonzero_words(ext)
            if col:
                st.col_nzw += _nonzero_words(ext)
        if parent[d] is not None:
            st.sum_c += size
            if bin(ctx.objects_of(parent[d])).count("1") > rowlocal_max:
                st.col_child_objs += size
    return st


def hasse_lower_covers(intents_in_order: list[int]) -> list[list[int]]:
    """The cover relation from the definition: for every concept i (intents as
    Python-int sets, in some fixed order) the positions j of the concepts right
    below it: B_i strictly inside B_j with no B_k strictly between."""
    below = [[j for j, d in enumerate(intents_in_order) if d != b and (b & ~d) == 0] for b in intents_in_order]
    out = []
    for i, js in enumerate(below):
        covers = []
        for j in js:
            dj = intents_in_order[j]
            if not any(k != j and (dk := intents_in_order[k]) != dj and (dk & ~dj) == 0 for k in js):
                covers.append(j)
        out.append(sorted(covers))
    return out
