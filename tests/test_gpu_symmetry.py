"""GPU results under the symmetries of the concept lattice (the oracle's own
tests check the same on the CPU): renaming the objects changes no intent,
renaming the attributes renames the intents, and the transposed context has
the same lattice with intents and extents exchanged.  These compare device
results with device results, so they pin the kernels independently of the
oracle; every input is also checked against the oracle's concept count.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import closed_set_enumeration_amd as fca  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fca.load_library()
    torch.cuda.set_device(0)


def run(cells):
    cells = np.asarray(cells, dtype=bool)
    rows = synth.pack_rows(cells)
    ctx = fca.Context(rows, cells.shape[1])
    try:
        res = ctx.enumerate(extents=True)
        torch.cuda.synchronize()
        ints = res.intents.cpu().numpy().view(np.uint64)
        exts = res.extents.cpu().numpy().view(np.uint64)
        conc, _ = ctx.level_counts()
        return res, ints, exts, [int(x) for x in conc]
    finally:
        ctx.close()


def as_sets(words, width):
    """Rows of bit words as frozensets of element indices."""
    out = []
    for r in words:
        s = []
        for w, v in enumerate(r):
            v = int(v)
            while v:
                b = v & -v
                s.append(64 * w + b.bit_length() - 1)
                v ^= b
        out.append(frozenset(e for e in s if e < width))
    return out


CASES = [("ctx64x16", None), ("random", (7001, 150, 70, 0.12)), ("random", (7002, 90, 130, 0.08))]


def cells_of(case):
    name, spec = case
    if name != "random":
        return synth.make_config(name, packed=False)
    return synth.random_context(*spec)


@pytest.mark.parametrize("case", CASES)
def test_renaming_objects_changes_no_intent(case):
    cells = cells_of(case)
    n, m = cells.shape
    perm = np.random.default_rng(11).permutation(n)  # new object i is old object perm[i]
    a, ia, ea, ca = run(cells)
    b, ib, eb, cb = run(cells[perm])
    assert a.n_concepts == b.n_concepts == oracle.cbo(synth.pack_rows(cells), m).n_concepts
    # same intents in the same order, same tests and levels
    assert np.array_equal(ia, ib)
    assert a.stats["closure_tests"] == b.stats["closure_tests"] and ca == cb
    # extents: the same sets of objects under the renaming
    inv = np.empty(n, dtype=np.int64)
    inv[perm] = np.arange(n)
    for sa, sb in zip(as_sets(ea, n), as_sets(eb, n)):
        assert sb == frozenset(int(inv[g]) for g in sa)


@pytest.mark.parametrize("case", CASES)
def test_renaming_attributes_renames_the_intents(case):
    cells = cells_of(case)
    n, m = cells.shape
    perm = np.random.default_rng(12).permutation(m)  # new attribute j is old attribute perm[j]
    a, ia, ea, _ = run(cells)
    b, ib, eb, _ = run(cells[:, perm])
    assert a.n_concepts == b.n_concepts
    want = dict(zip(as_sets(ia, m), as_sets(ea, n)))
    got = {frozenset(int(perm[j]) for j in s): e for s, e in zip(as_sets(ib, m), as_sets(eb, n))}
    assert got == want


@pytest.mark.parametrize("case", CASES)
def test_the_transposed_context_exchanges_intents_and_extents(case):
    cells = cells_of(case)
    n, m = cells.shape
    a, ia, ea, _ = run(cells)
    t, it, et, _ = run(cells.T)
    assert a.n_concepts == t.n_concepts
    pairs = set(zip(as_sets(ea, n), as_sets(ia, m)))        # (extent, intent) of the context
    pairs_t = set(zip(as_sets(it, n), as_sets(et, m)))      # (intent, extent) of the transpose
    assert pairs == pairs_t
