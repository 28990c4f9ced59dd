"""GPU cover edges (fcbo_cover_edges) against the CPU oracle, edge for edge.

The oracle (oracle/cover.c) takes the minimal closures (B + {m})'' of every
concept and is pinned against the Hasse diagram built from the definition; the
GPU kernels decide covers by object counts (a closure is a cover when all its
attributes outside B have the same object count).  Both list, per concept in
output order, its lower covers' output positions in ascending order.
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


def assert_cover_parity(cells, flags=0):
    cells = np.asarray(cells, dtype=bool)
    rows = synth.pack_rows(cells)
    m = cells.shape[1]
    want = oracle.cbo(rows, m, keep_extents=False)
    w_off, w_tg = oracle.cover_edges(rows, m, want.intents)
    ctx = fca.Context(rows, m, flags=flags)
    try:
        assert ctx.count() == want.n_concepts
        off, tg, _ = ctx.cover_edges()
        torch.cuda.synchronize()
        assert np.array_equal(off.cpu().numpy(), w_off)
        assert np.array_equal(tg.cpu().numpy().astype(np.int64), w_tg)
        # a second call gives the same bytes; too small a buffer gives the count only
        off2, tg2, _ = ctx.cover_edges()
        assert torch.equal(off, off2) and torch.equal(tg, tg2)
        e = len(w_tg)
        if e > 0:
            small = torch.full((e - 1 if e > 1 else 1,), -9, dtype=torch.int32, device="cuda")
            o = torch.full((want.n_concepts + 1,), -9, dtype=torch.int64, device="cuda")
            rc, e_seen, _ = fca.fcbo_cover_edges(ctx.handle, o.data_ptr(), small.data_ptr(), e - 1)
            assert rc == fca.FCBO_ERR_CAPACITY and e_seen == e
            assert bool((small == -9).all()) and bool((o == -9).all())
    finally:
        ctx.close()
    return w_off, w_tg


@pytest.mark.parametrize("name", ["ctx64x16", "ctx2000x64", "ctx10000x128"])
@pytest.mark.parametrize("flags", [0, fca.FCBO_TINY_BUFFERS])
def test_seeded_contexts(name, flags):
    # The counting pass keeps every cover's position for the writing call; with
    # tiny buffers that room runs out part-way, and the writing call takes a
    # second pass over the concepts instead.
    assert_cover_parity(synth.make_config(name, packed=False), flags=flags)


@pytest.mark.parametrize("n,m", [(1, 1), (63, 65), (65, 64), (129, 127), (200, 129)])
def test_edge_shapes(n, m):
    assert_cover_parity(synth.random_context(313 * n + m, n, m, min(0.4, 6.0 / m)))


@pytest.mark.parametrize("k", [2, 65, 130])
def test_diagonal(k):
    _, tg = assert_cover_parity(synth.diagonal(k))
    assert len(tg) == 2 * k


def test_contranominal_padded_multiword():
    _, tg = assert_cover_parity(synth.pad_with_full(synth.contranominal(11), extra_objects=118, extra_attrs=58))
    assert len(tg) == 11 * 2 ** 10


@pytest.mark.parametrize("n,m", [(70, 5), (200, 130)])
def test_trivial_lattices(n, m):
    _, tg = assert_cover_parity(synth.all_zero(n, m))
    assert len(tg) == 1
    _, tg = assert_cover_parity(synth.all_ones(n, m))
    assert len(tg) == 0


def test_large_extents_and_duplicate_rows():
    # concepts of 65..70,000 objects (the workgroup kernel), with rows repeated
    # so that some large extents share one row (their only cover is the bottom)
    cells = synth.random_context(4401, 20000, 24, 0.08)
    cells[5000:5100] = cells[4999]
    assert_cover_parity(cells)
    assert_cover_parity(synth.random_context(4402, 70000, 16, 0.1))


@pytest.mark.parametrize("m", [300, 447, 512])
def test_five_to_eight_word_intents(m):
    cells = synth.random_context(7 * m, 700, m, 0.03)
    rng = np.random.default_rng(m)
    for a in rng.choice(m, 5, replace=False):
        cells[:, a] |= rng.random(700) < 0.5
    assert_cover_parity(cells)


@pytest.mark.parametrize("n,m,d", [(40, 600, 0.01), (70, 1100, 0.004), (20, 4096, 0.001)])
def test_wide_attribute_sets(n, m, d):
    # more than 8 intent words: every concept takes the workgroup kernel
    assert_cover_parity(synth.random_context(n * m + 1, n, m, d))


@pytest.mark.parametrize("extra", [3, 70])
def test_a_million_concepts_keep_the_positions(extra):
    # 2^20 concepts (the contranominal scale of 20, padded across intent
    # words): from that size on the counting pass keeps every cover's position
    # and the writing call only copies them; with 70 full objects added every
    # extent has more than 64 objects and the workgroup kernel does it all.
    # The Boolean lattice of 20 atoms has 20 * 2^19 cover edges.
    cells = synth.pad_with_full(synth.contranominal(20), extra_objects=extra, extra_attrs=50)
    _, tg = assert_cover_parity(cells)
    assert len(tg) == 20 * 2 ** 19


from tests.test_gpu_parity import SWEEP, _planted  # noqa: E402


@pytest.mark.parametrize("seed,n,m,d,b", SWEEP)
def test_random_shapes_with_planted_blocks(seed, n, m, d, b):
    # up to eleven intent words (the wide-intent cover kernels at 700 attributes)
    assert_cover_parity(_planted(seed, n, m, d, b))
