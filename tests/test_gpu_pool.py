"""GPU parity of the task-pool schedule (FCBO_TASK_POOL).

With the flag the level loop expands only the parents with more than 16
objects and the subtrees of all other concepts are enumerated depth-first, one
task per wavefront.  The result must be the one the oracle gives, bit for bit:
concept count, ordered intents and extents, closure tests, item pairs, the
per-level numbers and the byte-model counters; the output API (paging, host
copies) and the cover edges work on a pool result as on any other.
"""

import hashlib
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import intent_digest as dg
from tests.conftest import release_device_cache
from tests.golden_io import read_fixture

torch = pytest.importorskip("torch")
import closed_set_enumeration_amd as fca  # noqa: E402

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fca.load_library()
    torch.cuda.set_device(0)


def pool_parity(cells, extents=True, ctx_flags=0):
    cells = np.asarray(cells, dtype=bool)
    rows = synth.pack_rows(cells)
    m = cells.shape[1]
    want = oracle.cbo(rows, m, keep_extents=extents)
    ctx = fca.Context(rows, m, flags=ctx_flags)
    try:
        res = ctx.enumerate(extents=extents, pool=True)
        conc, tests = ctx.level_counts()
        st = res.stats
        assert res.n_concepts == want.n_concepts
        assert np.array_equal(res.intents.cpu().numpy().view(np.uint64), want.intents)
        if extents:
            assert np.array_equal(res.extents.cpu().numpy().view(np.uint64), want.extents)
        assert st["closure_tests"] == want.tests
        assert st["item_pairs"] == want.pairs
        assert st["sum_child_objects"] == want.sum_c
        assert [int(x) for x in conc] == [int(x) for x in want.level_concepts]
        assert [int(x) for x in tests] == [int(x) for x in want.level_tests]
        assert st["local_parent_objects"] + st["medium_parent_objects"] == want.sum_rl_objs
        assert st["big_parents"] == want.col_parents
        assert st["big_nonzero_words"] == want.col_nzw
        assert st["big_child_objects"] == want.col_child_objs
        assert st["model_bytes"] == oracle.model_bytes(want)
        return res, want
    finally:
        ctx.close()


@pytest.mark.parametrize("name", ["staircase4.txt", "two_blocks4.txt"])
def test_hand_derived_examples(name):
    cells, _, info = read_fixture(name)
    res, _ = pool_parity(cells)
    assert res.n_concepts == info["concepts"]


@pytest.mark.parametrize("name", ["ctx64x16", "ctx2000x64", "ctx10000x128"])
@pytest.mark.parametrize("flags", [0, fca.FCBO_TINY_BUFFERS])
def test_seeded_contexts(name, flags):
    # tiny buffers: the pool's slots start at 64 and overflow, so the pool runs
    # again with twice as many until it fits
    pool_parity(synth.make_config(name, packed=False), ctx_flags=flags)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 129])
@pytest.mark.parametrize("m", [1, 64, 65, 130])
def test_edge_shapes(n, m):
    density = min(0.4, 6.0 / m)
    pool_parity(synth.random_context(10007 * n + m, n, m, density))


@pytest.mark.parametrize("m,d", [(300, 0.05), (447, 0.04), (512, 0.035)])
def test_five_to_eight_word_intents(m, d):
    cells = synth.random_context(7919 * m + 1000, 1000, m, d)
    rng = np.random.default_rng(m)
    for a in rng.choice(m, 6, replace=False):
        cells[:, a] |= rng.random(1000) < 0.6
    pool_parity(cells)


def test_special_contexts():
    for cells, k in [(synth.all_zero(65, 130), 2), (synth.all_ones(129, 3), 1), (synth.diagonal(65), 67),
                     (synth.diagonal(130), 132)]:
        res, _ = pool_parity(cells)
        assert res.n_concepts == k
    # 2^12 concepts, a task of 12 objects whose subtree is every subset (depth 12)
    res, _ = pool_parity(synth.pad_with_full(synth.contranominal(12), extra_objects=118, extra_attrs=58))
    assert res.n_concepts == 4096


def test_deepest_task_subtree():
    # the contranominal scale of 16 objects padded with full columns: the root
    # has 16 objects, the largest pool task, and the pool's descent reaches
    # depth 16 below it (all 2^16 concepts in one task); the same scale under
    # 48 more objects, where the level loop expands the root and the tasks
    # start lower
    res, _ = pool_parity(synth.pad_with_full(synth.contranominal(16), extra_attrs=20), extents=False)
    assert res.n_concepts == 65536
    res, _ = pool_parity(synth.pad_with_full(synth.contranominal(16), extra_objects=48, extra_attrs=20),
                         extents=False)
    assert res.n_concepts == 65536


def test_more_than_512_attributes_is_refused():
    cells = synth.random_context(3, 100, 513, 0.02)
    ctx = fca.Context(synth.pack_rows(cells), 513)
    try:
        with pytest.raises(fca.FcboError) as e:
            ctx.count(pool=True)
        assert e.value.code == fca.FCBO_ERR_INVALID_ARGUMENT
    finally:
        ctx.close()


def test_output_paging_host_copy_and_cover_edges_on_a_pool_result():
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 64, keep_extents=True)
    ctx = fca.Context(rows, 64)
    try:
        k = ctx.count(pool=True)
        assert k == want.n_concepts
        # pages of the ordered output
        buf_i = torch.empty((10007, 1), dtype=torch.int64, device="cuda")
        buf_e = torch.empty((10007, 32), dtype=torch.int64, device="cuda")
        for first in range(0, k, 10007):
            cnt = min(10007, k - first)
            ctx.write_range(first, intents=buf_i[:cnt], extents=buf_e[:cnt])
            assert np.array_equal(buf_i[:cnt].cpu().numpy().view(np.uint64), want.intents[first:first + cnt])
            assert np.array_equal(buf_e[:cnt].cpu().numpy().view(np.uint64), want.extents[first:first + cnt])
        hi = np.zeros((k, 1), dtype=np.uint64)
        ctx.copy_to_host(0, k, intents=hi, staging_rows=4096)
        assert np.array_equal(hi, want.intents)
        # lattice cover edges of the pool result against the oracle's
        offsets, targets, _ = ctx.cover_edges()
        off_w, tg_w = oracle.cover_edges(rows, 64, want.intents)
        assert np.array_equal(offsets.cpu().numpy(), off_w)
        assert np.array_equal(targets.cpu().numpy().astype(np.int64), tg_w)
    finally:
        ctx.close()


def test_pool_then_level_sync_on_one_context():
    cells = synth.make_config("ctx10000x128", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 128, keep_extents=False)
    ctx = fca.Context(rows, 128)
    try:
        for pool in (True, False, True):
            res = ctx.enumerate(extents=False, pool=pool)
            assert np.array_equal(res.intents.cpu().numpy().view(np.uint64), want.intents)
            assert res.stats["closure_tests"] == want.tests
    finally:
        ctx.close()


def test_pool_out_of_memory_leaves_a_usable_context():
    # A pool run that crosses the memory limit fails with FCBO_ERR_OUT_OF_MEMORY,
    # keeps no result and releases its buffers; the same context then
    # enumerates correctly with either schedule.
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 64, keep_extents=False)
    ctx = fca.Context(rows, 64, flags=fca.FCBO_TINY_BUFFERS)
    try:
        ints, _ = ctx.alloc_outputs(want.n_concepts, extents=False)
        rc, k, st = ctx.enumerate_into(ints, None, fca.FCBO_TASK_POOL)
        assert rc == fca.FCBO_OK and k == want.n_concepts
        ctx.set_memory_limit(st["peak_device_bytes"] * 9 // 10)  # releases what the run held
        with pytest.raises(fca.FcboError) as e:
            ctx.enumerate_into(ints, None, fca.FCBO_TASK_POOL)
        assert e.value.code == fca.FCBO_ERR_OUT_OF_MEMORY
        with pytest.raises(fca.FcboError):
            ctx.level_counts()
        ctx.set_memory_limit(0)
        for flags in (0, fca.FCBO_TASK_POOL):
            ints.fill_(-1)
            rc, k, st = ctx.enumerate_into(ints, None, flags)
            assert rc == fca.FCBO_OK and k == want.n_concepts
            assert np.array_equal(ints.cpu().numpy().view(np.uint64), want.intents)
            assert st["closure_tests"] == want.tests
    finally:
        ctx.close()


def test_full_ctx50000x400_pool_against_stored_oracle():
    release_device_cache()
    path = os.path.join(GOLDEN, "ctx50000x400.json")
    if not os.path.exists(path):
        pytest.skip("stored oracle values not generated")
    g = json.load(open(path))
    rows = synth.make_config("ctx50000x400")
    assert synth.rows_sha256(rows) == g["rows_sha256"]
    ctx = fca.Context(rows, 400)
    try:
        res = ctx.enumerate(extents=True, pool=True)
        st = res.stats
        conc, tests = ctx.level_counts()
        assert res.n_concepts == g["n_concepts"]
        assert st["closure_tests"] == g["closure_tests"]
        assert st["item_pairs"] == g["item_pairs"]
        assert st["sum_child_objects"] == g["sum_c"]
        assert st["model_bytes"] == g["model_bytes"]
        assert [int(x) for x in conc] == g["level_concepts"]
        assert [int(x) for x in tests] == g["level_tests"]
        ints = res.intents.cpu().numpy().view(np.uint64)
        assert hashlib.sha256(np.ascontiguousarray(ints, dtype="<u8").tobytes()).hexdigest() == g["intents_sha256"]
        eh = dg.extent_hashes_torch(res.extents).cpu().numpy().view(np.uint64)
        assert hashlib.sha256(np.ascontiguousarray(eh, dtype="<u8").tobytes()).hexdigest() == g["extent_hashes_sha256"]
    finally:
        ctx.close()


from tests.test_gpu_parity import SWEEP, _planted  # noqa: E402


@pytest.mark.parametrize("seed,n,m,d,b", [c for c in SWEEP if c[2] <= 512])
def test_random_shapes_with_planted_blocks(seed, n, m, d, b):
    pool_parity(_planted(seed, n, m, d, b))
