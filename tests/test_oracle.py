"""Pins of the CPU oracle (oracle/cbo.c) against what the mathematics fixes.

Nothing here touches the GPU library.  Every check compares the serial CbO
oracle with something other than itself:
  * hand-derived worked examples (tests/golden/*.txt),
  * two brute-force enumerations from the definition of a concept
    (all 2^M attribute subsets closed; all intersections of object rows),
  * the CbO generation tree reconstructed from the closed sets alone, which
    pins the closure-test count, item pairs, per-level counts and byte sums,
  * closed forms (empty, full, diagonal, contranominal, one bicluster),
  * invariances (duality, permutations, full rows/columns) and closedness
    checked with numpy on the 0/1 matrix.
"""

import itertools
from math import comb

import numpy as np
import pytest

import oracle
import synth
from oracle import brute
from tests.golden_io import read_fixture


def run(cells, keep_extents=True):
    cells = np.asarray(cells, dtype=bool)
    return oracle.cbo(synth.pack_rows(cells), cells.shape[1], keep_extents=keep_extents)


def as_sets(words):
    """uint64 [K, W] -> list of Python-int sets (in the given order)."""
    out = []
    for row in np.asarray(words, dtype=np.uint64):
        v = 0
        for w, x in enumerate(row):
            v |= int(x) << (64 * w)
        out.append(v)
    return out


def check_against_brute(cells, tree=True, subsets=None):
    ctx = brute.Context(cells)
    fam = brute.closed_intents_by_row_meets(ctx)
    if subsets is None:
        subsets = ctx.m <= 10
    if subsets:
        assert brute.closed_intents_by_subsets(ctx) == fam
    r = run(cells)
    ti, te = brute.sorted_concepts(ctx, fam)
    assert r.n_concepts == len(fam)
    assert np.array_equal(r.intents, ti)
    assert np.array_equal(r.extents, te)
    assert r.saturation_violations == 0
    assert not r.truncated
    if tree:
        st = brute.cbo_tree(ctx, fam)
        assert r.tests == st.tests
        assert r.pairs == st.pairs
        assert list(r.level_concepts) == st.level_concepts
        assert list(r.level_tests) == st.level_tests
        assert r.sum_nzw == st.sum_nzw
        assert r.sum_c == st.sum_c
        assert as_sets(r.intents) == preorder_descending(st)
    return r


def preorder_descending(st):
    """Intents of the CbO tree in pre-order, children visited by descending cursor."""
    kids = {}
    top = None
    for d, p in st.parent.items():
        if p is None:
            top = d
        else:
            kids.setdefault(p, []).append(d)
    out, stack = [], [top]
    while stack:
        d = stack.pop()
        out.append(d)
        # push ascending so that the largest cursor is popped first
        stack.extend(sorted(kids.get(d, []), key=lambda c: st.cursor[c]))
    return out


# --- worked examples -----------------------------------------------------------

@pytest.mark.parametrize("name", ["staircase4.txt", "two_blocks4.txt"])
def test_hand_derived_examples(name):
    cells, concepts, info = read_fixture(name)
    r = run(cells)
    assert r.n_concepts == info["concepts"]
    assert r.tests == info["tests"]
    assert r.pairs == info["pairs"]
    assert list(r.level_concepts) == info["level_concepts"]
    assert list(r.level_tests) == info["level_tests"]
    want_i = synth.pack_rows(np.array([c[0] for c in concepts]))
    want_e = synth.pack_rows(np.array([c[1] for c in concepts]))
    assert np.array_equal(r.intents, want_i)
    assert np.array_equal(r.extents, want_e)


# --- brute force -------------------------------------------------------------------

def test_ctx64x16_against_all_subsets():
    cells = synth.make_config("ctx64x16", packed=False)
    r = check_against_brute(cells, tree=True, subsets=True)
    assert r.n_concepts == 419


def test_random_tiny_contexts_against_brute_force():
    rng = np.random.default_rng(12345)
    n_cases = 0
    for case in range(520):
        n = int(rng.integers(1, 71))
        m = int(rng.integers(1, 15))
        density = float(rng.uniform(0.05, 0.95))
        cells = synth.random_context(1000 + case, n, m, density)
        ctx = brute.Context(cells)
        fam = brute.closed_intents_by_row_meets(ctx)
        check_against_brute(cells, tree=len(fam) <= 1500, subsets=m <= 8)
        n_cases += 1
    assert n_cases >= 500


def test_multiword_random_against_row_meets():
    # shapes that cross 64-bit word boundaries in both directions
    for seed, (n, m, d) in enumerate([(65, 66, 0.04), (130, 70, 0.03), (64, 129, 0.02), (127, 64, 0.05)]):
        cells = synth.random_context(77 + seed, n, m, d)
        check_against_brute(cells, tree=True, subsets=False)


# --- closed forms --------------------------------------------------------------------

@pytest.mark.parametrize("n,m", [(1, 1), (5, 3), (64, 64), (65, 130)])
def test_all_zero_context_has_top_and_bottom(n, m):
    r = run(synth.all_zero(n, m))
    assert r.n_concepts == 2  # (G, {}) and ({}, M)
    assert as_sets(r.intents) == [0, (1 << m) - 1]


@pytest.mark.parametrize("n,m", [(1, 1), (7, 70), (130, 3)])
def test_all_ones_context_has_one_concept(n, m):
    r = run(synth.all_ones(n, m))
    assert r.n_concepts == 1
    assert r.tests == 0
    assert as_sets(r.extents) == [(1 << n) - 1]


@pytest.mark.parametrize("k", [2, 3, 10, 64, 65, 100])
def test_diagonal_context(k):
    r = run(synth.diagonal(k))
    assert r.n_concepts == k + 2
    want = sorted([0, (1 << k) - 1] + [1 << i for i in range(k)])
    got = as_sets(r.intents)
    assert sorted(got) == want


@pytest.mark.parametrize("k", [1, 2, 5, 8, 11])
def test_contranominal_every_subset_closed(k):
    r = run(synth.contranominal(k))
    assert r.n_concepts == 2 ** k
    # every closure test passes, so tests = K - 1; level d holds C(k, d) sets
    assert r.tests == 2 ** k - 1
    assert list(r.level_concepts) == [comb(k, d) for d in range(k + 1)]


def test_contranominal_padded_across_words():
    k = 12
    cells = synth.pad_with_full(synth.contranominal(k), extra_objects=118, extra_attrs=58)  # 130 x 70
    r = run(cells)
    assert r.n_concepts == 2 ** k
    assert r.tests == 2 ** k - 1
    pad = sum(1 << a for a in range(k, k + 58))
    assert set(as_sets(r.intents)) == {s | pad for s in range(2 ** k)}


def test_single_planted_bicluster():
    cells = synth.planted_bicluster(50, 20, objs=[3, 7, 11, 40], atts=[2, 5, 19])
    r = run(cells)
    assert r.n_concepts == 3
    assert as_sets(r.intents) == [0, (1 << 2) | (1 << 5) | (1 << 19), (1 << 20) - 1]


def test_full_rows_and_columns_leave_concepts_unchanged():
    cells = synth.random_context(5, 40, 12, 0.35)
    base = run(cells)
    padded = run(synth.pad_with_full(cells, extra_objects=3, extra_attrs=0))
    assert padded.n_concepts == base.n_concepts
    assert np.array_equal(padded.intents, base.intents)
    more = run(synth.pad_with_full(cells, extra_objects=0, extra_attrs=2))
    assert more.n_concepts == base.n_concepts


# --- invariances -------------------------------------------------------------------------

def test_duality_ctx64x16():
    cells = synth.make_config("ctx64x16", packed=False)
    r = run(cells)
    rt = run(cells.T)
    assert rt.n_concepts == r.n_concepts
    assert set(as_sets(rt.intents)) == set(as_sets(r.extents))
    assert set(as_sets(rt.extents)) == set(as_sets(r.intents))


def test_duality_random():
    for seed in range(20):
        cells = synth.random_context(300 + seed, 30, 25, 0.3)
        r, rt = run(cells), run(cells.T)
        assert rt.n_concepts == r.n_concepts
        assert set(as_sets(rt.intents)) == set(as_sets(r.extents))


def test_object_permutation_keeps_intents():
    cells = synth.make_config("ctx64x16", packed=False)
    perm = np.random.default_rng(9).permutation(cells.shape[0])
    r, rp = run(cells), run(cells[perm])
    assert np.array_equal(r.intents, rp.intents)


def test_attribute_permutation_permutes_intents():
    cells = synth.make_config("ctx64x16", packed=False)
    perm = np.random.default_rng(10).permutation(cells.shape[1])
    r, rp = run(cells), run(cells[:, perm])
    assert rp.n_concepts == r.n_concepts
    # attribute perm[i] of the original is attribute i of the permuted context
    mapped = set()
    for b in as_sets(rp.intents):
        mapped.add(sum(1 << int(perm[i]) for i in range(cells.shape[1]) if (b >> i) & 1))
    assert mapped == set(as_sets(r.intents))


# --- invariants on the larger seeded contexts ----------------------------------------

def _check_invariants(cells, r, sample=2000, seed=0):
    n, m = cells.shape
    k = r.n_concepts
    ints = r.intents
    # strictly increasing in lexicographic order over attributes 0..m-1: at the
    # first attribute where neighbours differ, the later one has it
    ib = synth.unpack_rows(ints, m)
    if k > 1:
        ne = ib[1:] != ib[:-1]
        assert ne.any(axis=1).all()
        first = ne.argmax(axis=1)
        assert ib[1:][np.arange(k - 1), first].all()
    top = cells.all(axis=0)
    assert (ib == top).all(axis=1).any()
    assert ib.all(axis=1).any()  # bottom intent M
    assert int(r.level_concepts.sum()) == k and r.level_concepts[0] == 1
    rng = np.random.default_rng(seed)
    idx = rng.choice(k, size=min(sample, k), replace=False)
    for i in idx:
        b = ib[i]
        ext = cells[:, b].all(axis=1)  # B'
        back = cells[ext].all(axis=0) if ext.any() else np.ones(m, dtype=bool)  # B''
        assert np.array_equal(back, b)
        if r.extents is not None:
            assert np.array_equal(synth.unpack_rows(r.extents[i:i + 1], n)[0], ext)


def test_invariants_ctx2000x64():
    cells = synth.make_config("ctx2000x64", packed=False)
    r = run(cells)
    _check_invariants(cells, r)
    # |A| summed over all concepts = |G| for the root + sum of |C| over children
    total = int(np.unpackbits(r.extents.view(np.uint8)).sum())
    assert total == cells.shape[0] + r.sum_c


def test_invariants_ctx10000x128():
    cells = synth.make_config("ctx10000x128", packed=False)
    r = run(cells, keep_extents=False)
    _check_invariants(cells, r, sample=1000)


@pytest.mark.parametrize("name,attrs", [("ctx2000x64", [0, 17, 63]), ("ctx10000x128", [3, 64, 127])])
def test_slices_match_subcontexts(name, attrs):
    """Intents containing j are exactly the intents of the objects having j."""
    cells = synth.make_config(name, packed=False)
    r = run(cells, keep_extents=False)
    ib = synth.unpack_rows(r.intents, cells.shape[1])
    for j in attrs:
        sub = cells[cells[:, j]]
        rs = run(sub, keep_extents=False)
        mine = r.intents[ib[:, j]]
        assert np.array_equal(rs.intents, mine)


def test_truncation_budget():
    cells = synth.make_config("ctx2000x64", packed=False)
    r = oracle.cbo(synth.pack_rows(cells), 64, keep_extents=False, max_tests=1000)
    assert r.truncated and r.tests == 1000


# --- the store-free oracle and the intent digest -----------------------------------

def test_splitmix_output_function_reference_values():
    # SplitMix64 seeded with 0 (state advanced by the golden gamma before each
    # output) starts with these three outputs in the reference implementation
    from tests import intent_digest as dg

    state, outs = 0, []
    for _ in range(3):
        outs.append(dg.mix_py(state))
        state = (state + dg.GOLDEN) & dg.MASK
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_digest_implementations_agree():
    from tests import intent_digest as dg

    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    a = rng.integers(0, 1 << 63, size=(257, 3), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    want = dg.digest_py(a)
    assert dg.digest_np(a, chunk=100) == want
    assert dg.digest_torch(torch.from_numpy(a.view(np.int64)), chunk=64) == want


@pytest.mark.parametrize("case", ["ctx64x16", "ctx2000x64", "multiword", "contranominal", "all_zero"])
def test_store_free_oracle_matches_the_stored_search(case):
    from tests import intent_digest as dg

    if case in ("ctx64x16", "ctx2000x64"):
        cells = synth.make_config(case, packed=False)
    elif case == "multiword":
        cells = synth.random_context(913, 300, 150, 0.05)
    elif case == "contranominal":
        cells = synth.pad_with_full(synth.contranominal(10), extra_objects=70, extra_attrs=60)
    else:
        cells = synth.all_zero(70, 65)
    rows = synth.pack_rows(cells)
    m = cells.shape[1]
    r = oracle.cbo(rows, m, keep_extents=False)
    for threads in (1, 3):
        d = oracle.cbo_digest(rows, m, threads=threads)
        assert d.n_concepts == r.n_concepts
        assert (d.tests, d.pairs, d.sum_c) == (r.tests, r.pairs, r.sum_c)
        assert list(d.level_concepts) == list(r.level_concepts)
        assert list(d.level_tests) == list(r.level_tests)
        assert d.digest == dg.digest_np(r.intents)
    if r.n_concepts <= 5000:
        assert d.digest == dg.digest_py(r.intents)


# --- byte-model class split, extent hashes, positional digests ---------------------------

def test_class_split_sums_against_the_cbo_tree():
    # the oracle's split of the byte-model sums at a threshold T on |A| against
    # the CbO tree rebuilt from the closed sets; several T so both classes occur
    rng = np.random.default_rng(2024)
    for case in range(60):
        n = int(rng.integers(2, 90))
        m = int(rng.integers(2, 12))
        cells = synth.random_context(5000 + case, n, m, float(rng.uniform(0.1, 0.8)))
        ctx = brute.Context(cells)
        fam = brute.closed_intents_by_row_meets(ctx)
        if len(fam) > 800:
            continue
        rows = synth.pack_rows(cells)
        for t in (0, 1, n // 3, n // 2, n):
            st = brute.cbo_tree(ctx, fam, rowlocal_max=t)
            r = oracle.cbo(rows, m, keep_extents=False, rowlocal_max=t)
            assert (r.sum_rl_objs, r.col_parents, r.col_nzw, r.col_child_objs) == (
                st.sum_rl_objs, st.col_parents, st.col_nzw, st.col_child_objs), (case, t)
    # every parent in exactly one class: the row-local objects plus the larger
    # parents' objects are all objects of all concepts (|G| + sum |C|)
    cells = synth.make_config("ctx2000x64", packed=False)
    r = oracle.cbo(synth.pack_rows(cells), 64, keep_extents=True, rowlocal_max=100)
    sizes = np.unpackbits(r.extents.view(np.uint8), axis=1).sum(axis=1)
    assert r.sum_rl_objs == int(sizes[sizes <= 100].sum())
    assert r.col_parents == int((sizes > 100).sum())
    assert r.sum_rl_objs + int(sizes[sizes > 100].sum()) == cells.shape[0] + r.sum_c


@pytest.mark.parametrize("shape", [(64, 16, 0.3), (130, 40, 0.1), (200, 70, 0.05), (2000, 30, 0.1)])
def test_extent_hashes_follow_the_sorted_extents(shape):
    from tests import intent_digest as dg

    n, m, d = shape
    cells = synth.random_context(31 * n + m, n, m, d)
    r = oracle.cbo(synth.pack_rows(cells), m, keep_extents=True, hash_extents=True)
    want = dg.extent_hashes_np(r.extents)
    assert np.array_equal(r.extent_hashes, want)
    for i in range(0, r.n_concepts, max(1, r.n_concepts // 40)):
        assert int(r.extent_hashes[i]) == dg.extent_hash_py(r.extents[i])


def test_extent_hash_distinguishes_word_order_and_bits():
    from tests import intent_digest as dg

    a = np.array([5, 0, 9], dtype=np.uint64)
    assert dg.extent_hash_py(a) != dg.extent_hash_py(a[[2, 1, 0]])
    b = a.copy()
    b[1] = np.uint64(1 << 63)
    assert dg.extent_hash_py(a) != dg.extent_hash_py(b)
    # a word's term is f(word ^ f(index)): the empty one-word extent
    assert dg.extent_hash_py(np.zeros(1, dtype=np.uint64)) == dg.mix_py(dg.mix_py(0))


@pytest.mark.parametrize("case", ["ctx64x16", "ctx2000x64", "multiword", "contranominal", "all_zero", "one_object"])
def test_positional_digests_of_the_store_free_oracle(case):
    from tests import intent_digest as dg

    if case in ("ctx64x16", "ctx2000x64"):
        cells = synth.make_config(case, packed=False)
    elif case == "multiword":
        cells = synth.random_context(917, 300, 150, 0.05)
    elif case == "contranominal":
        cells = synth.pad_with_full(synth.contranominal(9), extra_objects=70, extra_attrs=60)
    elif case == "all_zero":
        cells = synth.all_zero(70, 65)
    else:
        cells = synth.random_context(3, 1, 20, 0.5)
    rows = synth.pack_rows(cells)
    m = cells.shape[1]
    r = oracle.cbo(rows, m, keep_extents=True, hash_extents=True)
    hi = dg.intent_hashes_np(r.intents)
    he = dg.extent_hashes_np(r.extents)
    assert np.array_equal(he, r.extent_hashes)
    for threads in (1, 3):
        d = oracle.cbo_digest(rows, m, threads=threads)
        assert d.subtree_size == d.n_concepts == r.n_concepts
        assert d.intent_digest == d.digest == int(hi.sum(dtype=np.uint64))
        assert d.intent_positional == dg.positional_np(hi)
        assert d.extent_digest == int(he.sum(dtype=np.uint64))
        assert d.extent_positional == dg.positional_np(he)
        # the root's children's subtrees: consecutive ranges after the root, by
        # descending attribute, each starting with the child itself
        start = 1
        attrs = [c["attr"] for c in d.root_children]
        assert attrs == sorted(attrs, reverse=True)
        for c in d.root_children:
            sl = slice(start, start + c["size"])
            assert c["hi0"] == int(hi[sl].sum(dtype=np.uint64))
            assert c["hi1"] == dg.positional_np(hi[sl])
            assert c["he0"] == int(he[sl].sum(dtype=np.uint64))
            assert c["he1"] == dg.positional_np(he[sl])
            first = synth.unpack_rows(r.intents[start:start + 1], m)[0]
            assert first[c["attr"]]
            start += c["size"]
        assert start == r.n_concepts
    if r.n_concepts <= 3000:
        assert d.intent_positional == dg.positional_py(hi)
        assert d.extent_positional == dg.positional_py([dg.extent_hash_py(x) for x in r.extents])


def test_model_bytes_inputs_are_the_class_sums():
    # model_bytes is the byte count stated with fcbo_stats; its inputs are the
    # pinned counters above.  All-ones 3 x 2: one concept, the root, row-local.
    r = oracle.cbo(synth.pack_rows(synth.all_ones(3, 2)), 2, keep_extents=False)
    assert (r.n_concepts, r.sum_rl_objs, r.col_parents, r.sum_c) == (1, 3, 0, 0)
    # parent read (8 + 4 + 16) + 3 objects x (4 + 8) + root rows and list 3 x (8 + 4)
    assert oracle.model_bytes(r) == 28 + 36 + 36


# --- lattice cover edges ---------------------------------------------------------------

def _edges_as_lists(offsets, targets):
    return [list(targets[offsets[i]:offsets[i + 1]]) for i in range(len(offsets) - 1)]


def test_cover_edges_against_the_hasse_diagram():
    rng = np.random.default_rng(777)
    for case in range(150):
        n = int(rng.integers(1, 40))
        m = int(rng.integers(1, 11))
        cells = synth.random_context(9000 + case, n, m, float(rng.uniform(0.1, 0.9)))
        r = run(cells, keep_extents=False)
        off, tg = oracle.cover_edges(synth.pack_rows(cells), m, r.intents)
        want = brute.hasse_lower_covers(as_sets(r.intents))
        assert _edges_as_lists(off, tg) == want, case


@pytest.mark.parametrize("k", [2, 3, 10, 70])
def test_cover_edges_diagonal(k):
    # top -> each atom -> bottom
    cells = synth.diagonal(k)
    r = run(cells, keep_extents=False)
    off, tg = oracle.cover_edges(synth.pack_rows(cells), k, r.intents)
    assert len(tg) == 2 * k


@pytest.mark.parametrize("k", [1, 4, 9])
def test_cover_edges_contranominal(k):
    # the Boolean lattice of k atoms: k * 2^(k-1) edges, every set covers its k - |B| one-larger supersets
    cells = synth.contranominal(k)
    r = run(cells, keep_extents=False)
    off, tg = oracle.cover_edges(synth.pack_rows(cells), k, r.intents)
    assert len(tg) == k * 2 ** (k - 1)
    sets = as_sets(r.intents)
    for i, b in enumerate(sets):
        assert [sets[t] for t in tg[off[i]:off[i + 1]]] == sorted(
            [b | (1 << a) for a in range(k) if not (b >> a) & 1], key=lambda d: brute.intent_key(d, k))


def test_cover_edges_chain_and_trivial_lattices():
    # staircase: object i has attributes 0..i, the lattice is a chain
    n = 70
    cells = np.tril(np.ones((n, n), dtype=bool))
    r = run(cells, keep_extents=False)
    off, tg = oracle.cover_edges(synth.pack_rows(cells), n, r.intents)
    assert len(tg) == r.n_concepts - 1
    for cells, edges in [(synth.all_zero(5, 4), 1), (synth.all_ones(5, 4), 0)]:
        r = run(cells, keep_extents=False)
        off, tg = oracle.cover_edges(synth.pack_rows(cells), cells.shape[1], r.intents)
        assert len(tg) == edges


def test_cover_edges_invariants_ctx2000x64():
    cells = synth.make_config("ctx2000x64", packed=False)
    r = run(cells, keep_extents=False)
    off, tg = oracle.cover_edges(synth.pack_rows(cells), 64, r.intents)
    k = r.n_concepts
    deg = np.diff(off)
    ib = synth.unpack_rows(r.intents, 64)
    bottom = int(np.flatnonzero(ib.all(axis=1))[0])
    assert (deg[np.arange(k) != bottom] > 0).all() and deg[bottom] == 0
    hit = np.zeros(k, dtype=bool)
    hit[tg] = True
    assert not hit[0] and hit[1:].all()  # every concept but the top has an upper cover
    src = np.repeat(np.arange(k), deg)
    # each edge goes to a strictly larger intent (every source attribute kept)
    sample = np.random.default_rng(5).choice(len(tg), size=3000, replace=False)
    for e in sample:
        a, b = ib[src[e]], ib[tg[e]]
        assert (b | ~a).all() and (b != a).any()


# --- property-based: contexts drawn and shrunk by hypothesis ----------------------------

from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as hs  # noqa: E402


@hs.composite
def _contexts(draw, max_n=24, max_m=9):
    """A 0/1 context; hypothesis favours the edge structure random draws rarely
    give (empty and full rows, repeated rows and columns) and shrinks a failure
    to a minimal context."""
    n = draw(hs.integers(1, max_n))
    m = draw(hs.integers(1, max_m))
    bits = draw(hs.lists(hs.lists(hs.booleans(), min_size=m, max_size=m), min_size=n, max_size=n))
    return np.array(bits, dtype=bool)


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow], derandomize=True,
          database=None)
@given(_contexts())
def test_property_concepts_against_both_brute_forces(cells):
    # every closed set from all attribute subsets and from row meets, in the
    # output order, with the CbO tree's counts
    check_against_brute(cells, tree=True, subsets=True)


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow], derandomize=True,
          database=None)
@given(_contexts(max_n=16, max_m=8))
def test_property_cover_edges_against_the_hasse_diagram(cells):
    r = run(cells, keep_extents=False)
    off, tg = oracle.cover_edges(synth.pack_rows(cells), cells.shape[1], r.intents)
    assert _edges_as_lists(off, tg) == brute.hasse_lower_covers(as_sets(r.intents))
