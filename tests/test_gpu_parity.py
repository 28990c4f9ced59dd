"""GPU parity: libfcbo against the CPU oracle, bit for bit.

Every test calls the HIP path through the C ABI (closed_set_enumeration_amd
marshals arguments only) and compares with oracle/ on the same seeded input:
the concept count, the sorted intent array byte for byte, the extents, the
closure-test and item-pair counts and the per-level counts.  All of it is
integer work, so the bar is exact equality.
"""

import ctypes
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
from tests.intent_digest import digest_torch

torch = pytest.importorskip("torch")
import closed_set_enumeration_amd as fca  # noqa: E402

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gpu_run(rows, m, extents=True, flags=0):
    ctx = fca.Context(rows, m, flags=flags)
    try:
        res = ctx.enumerate(extents=extents)
        torch.cuda.synchronize()
        ints = res.intents.cpu().numpy().view(np.uint64)
        exts = res.extents.cpu().numpy().view(np.uint64) if extents else None
        conc, tests = ctx.level_counts()
        return res, ints, exts, conc, tests
    finally:
        ctx.close()


def assert_model_counters(st, want):
    """The byte-model inputs counted on the device equal the oracle's class sums."""
    assert st["local_parent_objects"] + st["medium_parent_objects"] == want.sum_rl_objs
    assert st["big_parents"] == want.col_parents
    assert st["big_nonzero_words"] == want.col_nzw
    assert st["big_child_objects"] == want.col_child_objs
    assert st["model_bytes"] == oracle.model_bytes(want)


def assert_parity(cells, extents=True, flags=0):
    cells = np.asarray(cells, dtype=bool)
    rows = synth.pack_rows(cells)
    m = cells.shape[1]
    want = oracle.cbo(rows, m, keep_extents=extents)
    res, ints, exts, conc, tests = gpu_run(rows, m, extents=extents, flags=flags)
    assert_model_counters(res.stats, want)
    assert res.n_concepts == want.n_concepts
    assert ints.shape == want.intents.shape
    assert np.array_equal(ints, want.intents)
    if extents:
        assert np.array_equal(exts, want.extents)
    assert res.stats["closure_tests"] == want.tests
    assert res.stats["item_pairs"] == want.pairs
    assert res.stats["sum_child_objects"] == want.sum_c
    assert [int(x) for x in conc] == [int(x) for x in want.level_concepts]
    assert [int(x) for x in tests] == [int(x) for x in want.level_tests]
    return res


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fca.load_library()
    torch.cuda.set_device(0)


# --- worked examples and the small seeded contexts ---------------------------------

@pytest.mark.parametrize("name", ["staircase4.txt", "two_blocks4.txt"])
def test_hand_derived_examples(name):
    cells, concepts, info = read_fixture(name)
    res = assert_parity(cells)
    assert res.n_concepts == info["concepts"]


@pytest.mark.parametrize("name", ["ctx64x16", "ctx2000x64", "ctx10000x128"])
@pytest.mark.parametrize("flags", [0, fca.FCBO_TINY_BUFFERS])
def test_seeded_contexts(name, flags):
    res = assert_parity(synth.make_config(name, packed=False), flags=flags)
    if flags & fca.FCBO_TINY_BUFFERS:
        # buffers start at their minimum: record buffers overflow and levels run again
        assert res.stats["level_redos"] >= 1
    else:
        assert res.stats["level_redos"] == 0


# --- edge shapes: word boundaries on both axes, ragged tails ---------------------------

EDGE = [1, 63, 64, 65, 127, 128, 129]


@pytest.mark.parametrize("n", EDGE)
@pytest.mark.parametrize("m", EDGE)
def test_edge_shapes(n, m):
    density = min(0.4, 6.0 / m)
    cells = synth.random_context(10007 * n + m, n, m, density)
    assert_parity(cells)


@pytest.mark.parametrize("m,d,flags", [(300, 0.05, 0), (380, 0.045, 0), (447, 0.04, 0), (512, 0.035, 0),
                                         (447, 0.04, fca.FCBO_TINY_BUFFERS)])
def test_five_to_eight_word_intents(m, d, flags):
    # Intents of 5, 6, 7 and 8 words (the kernels' templates for these widths
    # take 16-parent chunks in the local test).  1,000 objects with six dense
    # attributes (density 0.6) besides the sparse ones, so the levels hold
    # local, narrow mid (65..512 objects) and wide mid (513..4096) parents.
    cells = synth.random_context(7919 * m + 1000, 1000, m, d)
    rng = np.random.default_rng(m)
    for a in rng.choice(m, 6, replace=False):
        cells[:, a] |= rng.random(1000) < 0.6
    assert_parity(cells, flags=flags)


@pytest.mark.parametrize("n,m,d", [(40, 600, 0.01), (70, 1100, 0.004), (20, 4096, 0.001), (130, 520, 0.012)])
def test_wide_attribute_sets(n, m, d):
    # more than 8 intent words: the generic word-count kernels
    assert_parity(synth.random_context(n * m, n, m, d))


def test_many_objects():
    # large extents: big parents split into 64-word chunks of their extent bitmap
    assert_parity(synth.random_context(70024, 70000, 24, 0.08))
    assert_parity(synth.random_context(70040, 70000, 40, 0.05), flags=fca.FCBO_TINY_BUFFERS)


def test_over_a_million_objects_list_path():
    # more than 2^20 objects: big parents are scanned through their object lists,
    # and extent rows wider than the output kernel's LDS tile are written tile by tile
    assert_parity(synth.random_context(1100006, 1_100_000, 6, 0.3), extents=True)


@pytest.mark.parametrize("n,m", [(65, 130), (130, 5), (1, 1), (300, 64)])
def test_all_zero(n, m):
    # the bottom ({}, M) comes from a parent with more than 64 objects when n > 64
    res = assert_parity(synth.all_zero(n, m))
    assert res.n_concepts == 2


@pytest.mark.parametrize("n,m", [(129, 3), (1, 200), (64, 64)])
def test_all_ones(n, m):
    res = assert_parity(synth.all_ones(n, m))
    assert res.n_concepts == 1


@pytest.mark.parametrize("k", [65, 130])
def test_diagonal(k):
    res = assert_parity(synth.diagonal(k))
    assert res.n_concepts == k + 2


def test_contranominal_padded_multiword():
    cells = synth.pad_with_full(synth.contranominal(12), extra_objects=118, extra_attrs=58)
    res = assert_parity(cells)
    assert res.n_concepts == 4096


def test_contranominal_large():
    # 2^16 concepts, every closure test passes
    cells = synth.pad_with_full(synth.contranominal(16), extra_objects=60, extra_attrs=120)
    res = assert_parity(cells, extents=True)
    assert res.n_concepts == 65536
    assert res.stats["closure_tests"] == 65535


def test_big_parents_mixed_density():
    # dense columns keep many parents above 64 objects for several levels
    rng = np.random.default_rng(4242)
    p = rng.uniform(0.02, 0.6, size=90)
    cells = rng.random((700, 90)) < p[None, :]
    assert_parity(cells, flags=fca.FCBO_TINY_BUFFERS)


# --- interface behaviour ---------------------------------------------------------------

def test_columns_are_the_transpose():
    cells = synth.random_context(77, 200, 130, 0.1)
    ctx = fca.Context(synth.pack_rows(cells), 130)
    try:
        cols = ctx.columns()
    finally:
        ctx.close()
    assert np.array_equal(cols, synth.pack_rows(cells.T))


def test_device_rows_and_strided_dirty_rows():
    cells = synth.random_context(78, 150, 70, 0.12)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 70)
    # stride 3 words, junk in the padding word and in the bits past M
    dirty = np.full((150, 3), np.uint64(0xDEADBEEFDEADBEEF), dtype=np.uint64)
    dirty[:, :2] = rows
    dirty[:, 1] |= np.uint64(~((1 << 6) - 1) & ((1 << 64) - 1))
    res, ints, exts, _, _ = gpu_run(dirty, 70)
    assert np.array_equal(ints, want.intents) and np.array_equal(exts, want.extents)
    dev = torch.from_numpy(dirty.view(np.int64)).cuda()
    res, ints, exts, _, _ = gpu_run(dev, 70)
    assert np.array_equal(ints, want.intents) and np.array_equal(exts, want.extents)


def test_run_twice_is_byte_identical():
    rows = synth.make_config("ctx2000x64")
    ctx = fca.Context(rows, 64)
    try:
        a = ctx.enumerate()
        ai, ae = a.intents.clone(), a.extents.clone()
        b = ctx.enumerate()
        assert torch.equal(ai, b.intents) and torch.equal(ae, b.extents)
    finally:
        ctx.close()


def test_capacity_error_and_reuse():
    cells = synth.make_config("ctx64x16", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 16)
    k = want.n_concepts
    ctx = fca.Context(rows, 16)
    try:
        ints, exts = ctx.alloc_outputs(k, True)
        ints.fill_(-7)
        exts.fill_(-7)
        small_i, small_e = ints[: k - 1], exts[: k - 1]
        rc, k_seen, _ = ctx.enumerate_into(small_i, small_e)
        assert rc == fca.FCBO_ERR_CAPACITY and k_seen == k
        torch.cuda.synchronize()
        assert bool((ints == -7).all()) and bool((exts == -7).all())
        rc, k_seen, st = ctx.enumerate_into(ints, exts, fca.FCBO_REUSE_RESULT)
        assert rc == fca.FCBO_OK and k_seen == k
        got = ints.cpu().numpy().view(np.uint64)
        assert np.array_equal(got, want.intents)
        assert np.array_equal(exts.cpu().numpy().view(np.uint64), want.extents)
        # intents only
        rc, _, _ = ctx.enumerate_into(ints, None)
        assert rc == fca.FCBO_OK
        assert np.array_equal(ints.cpu().numpy().view(np.uint64), want.intents)
    finally:
        ctx.close()


def test_write_range_pages_the_output():
    # output rows fetched piece by piece through small buffers, ragged last piece
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 64)
    k = want.n_concepts
    ctx = fca.Context(rows, 64)
    try:
        assert ctx.count() == k
        got_i = np.zeros_like(want.intents)
        got_e = np.zeros_like(want.extents)
        piece = 7777
        bi, be = ctx.alloc_outputs(piece, True)
        for first in range(0, k, piece):
            cnt = min(piece, k - first)
            ctx.write_range(first, bi[:cnt], be[:cnt])
            got_i[first:first + cnt] = bi[:cnt].cpu().numpy().view(np.uint64)
            got_e[first:first + cnt] = be[:cnt].cpu().numpy().view(np.uint64)
        assert np.array_equal(got_i, want.intents)
        assert np.array_equal(got_e, want.extents)
        # one buffer at a time, from the middle
        ctx.write_range(1234, extents=be[:100])
        assert np.array_equal(be[:100].cpu().numpy().view(np.uint64), want.extents[1234:1334])
        ctx.write_range(k - 50, intents=bi[:50])
        assert np.array_equal(bi[:50].cpu().numpy().view(np.uint64), want.intents[k - 50:])
        with pytest.raises(fca.FcboError) as e:
            ctx.write_range(k - 49, intents=bi[:50])
        assert e.value.code == fca.FCBO_ERR_INVALID_ARGUMENT
        fca.fcbo_write_range(ctx.handle, k, 0, bi.data_ptr(), 0)  # empty range at the end
    finally:
        ctx.close()


def test_copy_to_host_through_two_staging_buffers():
    # the output streamed to host memory in bounded pieces, overlapping the
    # output kernels of one piece with the copy of the other
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 64)
    k = want.n_concepts
    ctx = fca.Context(rows, 64)
    try:
        assert ctx.count() == k
        hi = torch.full((k, ctx.wm), -1, dtype=torch.int64).pin_memory()
        he = torch.full((k, ctx.wn), -1, dtype=torch.int64).pin_memory()
        ctx.copy_to_host(0, k, hi, he, staging_rows=7777)  # ragged last piece
        assert np.array_equal(hi.numpy().view(np.uint64), want.intents)
        assert np.array_equal(he.numpy().view(np.uint64), want.extents)
        # pageable numpy arrays, a middle range, one buffer at a time
        a = np.zeros((1000, ctx.wm), dtype=np.uint64)
        ctx.copy_to_host(500, 1000, intents=a, staging_rows=1 << 20)
        assert np.array_equal(a, want.intents[500:1500])
        b = np.zeros((10, ctx.wn), dtype=np.uint64)
        ctx.copy_to_host(k - 10, 10, extents=b, staging_rows=1)
        assert np.array_equal(b, want.extents[k - 10:])
        for first, count, staging in [(k - 9, 10, 4), (0, 10, 0)]:
            with pytest.raises(fca.FcboError) as e:
                fca.fcbo_copy_to_host(ctx.handle, first, count, a.ctypes.data, 0, staging)
            assert e.value.code == fca.FCBO_ERR_INVALID_ARGUMENT
        with pytest.raises(ValueError):
            ctx.copy_to_host(0, 2000, intents=a)  # fewer rows than asked for
    finally:
        ctx.close()


def test_memory_limit_fails_part_way_and_leaves_no_stale_result():
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 64)
    k = want.n_concepts
    ctx = fca.Context(rows, 64, flags=fca.FCBO_TINY_BUFFERS)  # buffers grow level by level
    try:
        ints, exts = ctx.alloc_outputs(k, True)
        rc, kk, _ = ctx.enumerate_into(ints, exts)
        assert rc == fca.FCBO_OK and kk == k
        conc, _ = ctx.level_counts()
        # a cap below what the enumeration holds: the buffers and the result go
        ctx.set_memory_limit(1 << 20)
        with pytest.raises(fca.FcboError):
            ctx.level_counts()
        for _ in range(2):
            ints.fill_(-5)
            exts.fill_(-5)
            with pytest.raises(fca.FcboError) as e:
                ctx.enumerate_into(ints, exts, fca.FCBO_REUSE_RESULT)
            assert e.value.code == fca.FCBO_ERR_OUT_OF_MEMORY
            torch.cuda.synchronize()
            assert bool((ints == -5).all()) and bool((exts == -5).all())  # nothing stale written
            with pytest.raises(fca.FcboError):
                ctx.level_counts()
        ctx.set_memory_limit(0)
        rc, kk, st = ctx.enumerate_into(ints, exts, fca.FCBO_REUSE_RESULT)
        assert rc == fca.FCBO_OK and kk == k
        assert np.array_equal(ints.cpu().numpy().view(np.uint64), want.intents)
        assert np.array_equal(exts.cpu().numpy().view(np.uint64), want.extents)
        assert [int(x) for x in ctx.level_counts()[0]] == [int(x) for x in conc]
    finally:
        ctx.close()


def test_failed_device_allocation_leaves_no_error_behind():
    # A context whose rows alone need ~1.1 TB: the row allocation fails (a real
    # hipMalloc failure, not the memory limit) and the call returns
    # FCBO_ERR_OUT_OF_MEMORY before it reads its input.  The HIP error of that
    # allocation must not surface in later calls as their own.
    n, m = (1 << 31) - 1, 4096
    need = n * (m // 64) * 8
    _, total = torch.cuda.mem_get_info()
    assert need > 2 * total
    with pytest.raises(torch.OutOfMemoryError):  # the device cannot hold it: nothing below can run
        torch.empty(need // 8, dtype=torch.int64, device="cuda")
    release_device_cache()
    small = torch.zeros(64, dtype=torch.int64, device="cuda")
    with pytest.raises(fca.FcboError) as e:
        fca.fcbo_context_create(small.data_ptr(), n, m, m // 64, fca.FCBO_ROWS_ON_DEVICE, 0)
    assert e.value.code == fca.FCBO_ERR_OUT_OF_MEMORY
    assert_parity(synth.make_config("ctx64x16", packed=False))


def test_output_buffers_are_checked_before_any_launch():
    rows = synth.make_config("ctx64x16")
    ctx = fca.Context(rows, 16)
    try:
        k = ctx.count()
        ints, exts = ctx.alloc_outputs(k, True)
        for bad_i, bad_e in [(ints[:, :0], exts), (ints.float(), exts),
                             (ints.t(), exts), (ints.cpu(), exts), (ints, exts.view(-1)[:k])]:
            with pytest.raises(ValueError):
                ctx.enumerate_into(bad_i, bad_e)
        # capacity is the smaller of the two buffers
        rc, kk, _ = ctx.enumerate_into(ints, exts[: k - 1])
        assert rc == fca.FCBO_ERR_CAPACITY and kk == k
    finally:
        ctx.close()


def test_fifty_thousand_objects_all_extents_compared():
    # N = 50,000 gives extent rows of 782 words, written eight rows per output
    # tile (the benchmark's tile shape); every row compared
    cells = synth.random_context(50020, 50_000, 20, 0.05)
    res = assert_parity(cells, extents=True)
    assert res.n_concepts > 1000


@pytest.mark.parametrize("n", [129, 2000])
def test_extent_buffer_only_word_aligned(n):
    # an extent buffer starting 8 bytes past a 16-byte boundary: single-word stores
    cells = synth.random_context(79 + n, n, 40, 0.1)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 40)
    k, wn = want.n_concepts, (n + 63) // 64
    ctx = fca.Context(rows, 40)
    try:
        ints, _ = ctx.alloc_outputs(k, False)
        flat = torch.full((k * wn + 1,), -3, dtype=torch.int64, device="cuda")
        exts = flat[1:].view(k, wn)
        assert exts.data_ptr() % 16 == 8
        rc, k_seen, _ = ctx.enumerate_into(ints, exts)
        assert rc == fca.FCBO_OK and k_seen == k
        torch.cuda.synchronize()
        assert int(flat[0]) == -3
        assert np.array_equal(ints.cpu().numpy().view(np.uint64), want.intents)
        assert np.array_equal(exts.cpu().numpy().view(np.uint64), want.extents)
    finally:
        ctx.close()


def test_invalid_arguments():
    rows = synth.make_config("ctx64x16")
    ptr = rows.ctypes.data
    for n, m, stride, flags in [(0, 16, 1, 0), (64, 0, 1, 0), (64, 4097, 65, 0), (64, 130, 2, 0), (64, 16, 1, 8)]:
        with pytest.raises(fca.FcboError) as e:
            fca.fcbo_context_create(ptr, n, m, stride, flags, 0)
        assert e.value.code == fca.FCBO_ERR_INVALID_ARGUMENT
    h = fca.fcbo_context_create(ptr, 64, 16, 1, 0, torch.cuda.current_stream().cuda_stream)
    try:
        with pytest.raises(fca.FcboError):
            fca.fcbo_enumerate(h, 0, 0, 0, 64)  # unknown flag
        with pytest.raises(fca.FcboError):
            fca.fcbo_level_counts(h)  # nothing enumerated yet
    finally:
        fca.fcbo_destroy(h)


# --- full-size seeded workloads ----------------------------------------------------------

def _popcount_rows(t, chunk=1 << 16):
    lut = torch.tensor([bin(i).count("1") for i in range(256)], dtype=torch.int64, device=t.device)
    total = 0
    for s in range(0, t.shape[0], chunk):
        total += int(lut[t[s:s + chunk].contiguous().view(torch.uint8).long()].sum())
    return total


def _sample_extents_match(cells, ints, exts_t, sample, seed):
    n, m = cells.shape
    ib = synth.unpack_rows(ints, m)
    k = ints.shape[0]
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([[0, k - 1], rng.choice(k, size=min(sample, k), replace=False)]))
    got = exts_t[torch.from_numpy(idx).to(exts_t.device)].cpu().numpy().view(np.uint64)
    for r, i in enumerate(idx):
        b = ib[i]
        ext = cells[:, b].all(axis=1)  # B'
        back = cells[ext].all(axis=0) if ext.any() else np.ones(m, dtype=bool)  # B''
        assert np.array_equal(back, b), i
        assert np.array_equal(synth.unpack_rows(got[r:r + 1], n)[0], ext), i


def _say(msg):
    print("[full-size] %s" % msg, flush=True)


def test_full_ctx50000x400_against_stored_oracle():
    # The benchmark's configuration (extents written).  Stored oracle values:
    # counts, SHA-256 of the ordered intents and of the ordered extent hashes
    # (every one of the 4.9 million extent rows hashed on the device), and the
    # positional digests of the store-free oracle.
    release_device_cache()
    path = os.path.join(GOLDEN, "ctx50000x400.json")
    if not os.path.exists(path):
        pytest.skip("stored oracle values not generated")
    g = json.load(open(path))
    cells = synth.make_config("ctx50000x400", packed=False)
    rows = synth.pack_rows(cells)
    assert synth.rows_sha256(rows) == g["rows_sha256"]
    ctx = fca.Context(rows, 400)
    try:
        res = ctx.enumerate(extents=True)
        torch.cuda.synchronize()
        ints = res.intents.cpu().numpy().view(np.uint64)
        conc, tests = ctx.level_counts()
        assert res.n_concepts == g["n_concepts"]
        assert hashlib.sha256(np.ascontiguousarray(ints, dtype="<u8").tobytes()).hexdigest() == g["intents_sha256"]
        assert res.stats["closure_tests"] == g["closure_tests"]
        assert res.stats["item_pairs"] == g["item_pairs"]
        assert res.stats["sum_child_objects"] == g["sum_c"]
        assert [int(x) for x in conc] == g["level_concepts"]
        assert [int(x) for x in tests] == g["level_tests"]
        st = res.stats
        assert st["local_parent_objects"] + st["medium_parent_objects"] == g["sum_rl_objs"]
        assert (st["big_parents"], st["big_nonzero_words"], st["big_child_objects"]) == (
            g["col_parents"], g["col_nzw"], g["col_child_objs"])
        assert st["model_bytes"] == g["model_bytes"]
        _say("ctx50000x400: counts and intents match; hashing extents")
        eh = dg.extent_hashes_torch(res.extents)
        ehs = eh.cpu().numpy().view(np.uint64)
        assert hashlib.sha256(np.ascontiguousarray(ehs, dtype="<u8").tobytes()).hexdigest() == g["extent_hashes_sha256"]
        assert dg.positional_torch(eh) == int(g["extent_positional"])
        assert dg.positional_torch(dg.intent_hashes_torch(res.intents)) == int(g["intent_positional"])
        # extras: every extent bit accounted for (|G| for the root plus |C| of
        # every child), and sampled rows against B' and closedness
        assert _popcount_rows(res.extents) == 50000 + g["sum_c"]
        _sample_extents_match(cells, ints, res.extents, 300, 4)
    finally:
        ctx.close()


def _check_root_subtrees(g, hashes, which):
    """Every child of the root owns one consecutive output range, by descending
    attribute, with the stored size, hash sum and position-weighted hash sum."""
    start = 1
    lo = 2 if which == "intent" else 4
    for attr, size, *sums in g["root_children"]:
        part = hashes[start:start + size]
        assert (int(part.sum()) & dg.MASK) == int(sums[lo - 2]), (which, attr)
        assert dg.positional_torch(part) == int(sums[lo - 1]), (which, attr)
        start += size
    assert start == hashes.shape[0]


def _assert_lectic_increasing(ints, chunk=1 << 26):
    """Consecutive rows strictly increase in lexicographic order over the
    attributes: at the first attribute where two rows differ, the later row
    has it (checked on the device, chunk by chunk)."""
    k, w = ints.shape
    for s in range(0, k - 1, chunk):
        a = ints[s:min(s + chunk, k - 1)]
        b = ints[s + 1:min(s + chunk, k - 1) + 1]
        x = a ^ b
        nz = x != 0
        assert bool(nz.any(dim=1).all()), "equal neighbouring intents"
        first = nz.int().argmax(dim=1)  # first differing word
        xw = x.gather(1, first[:, None]).squeeze(1)
        bw = b.gather(1, first[:, None]).squeeze(1)
        low = xw & (-xw)  # lowest differing bit of that word
        assert bool(((bw & low) != 0).all()), "rows out of lexicographic order"


def test_full_ctx20000x256_against_store_free_oracle():
    # 1.4e9 concepts.  Intents: counts, per-level numbers, the order-free and
    # the positional intent digests, the root's subtrees as output ranges, the
    # lexicographic order and slices compared byte for byte.  Extents (3.5 TB in
    # all) are paged through a bounded buffer with fcbo_write_range and every
    # row hashed on the device: positional extent digest and the root's subtrees.
    release_device_cache()
    path = os.path.join(GOLDEN, "ctx20000x256.json")
    if not os.path.exists(path):
        pytest.skip("stored oracle values not generated")
    g = json.load(open(path))
    rows = synth.make_config("ctx20000x256")
    assert synth.rows_sha256(rows) == g["rows_sha256"]
    ctx = fca.Context(rows, 256)
    try:
        res = ctx.enumerate(extents=False)
        torch.cuda.synchronize()
        conc, tests = ctx.level_counts()
        k = res.n_concepts
        assert k == g["n_concepts"]
        assert res.stats["closure_tests"] == g["closure_tests"]
        assert res.stats["item_pairs"] == g["item_pairs"]
        assert res.stats["sum_child_objects"] == g["sum_c"]
        assert [int(x) for x in conc] == g["level_concepts"]
        assert [int(x) for x in tests] == g["level_tests"]
        ints = res.intents
        _say("ctx20000x256: counts match; hashing intents")
        step = 1 << 27
        ih = torch.empty(k, dtype=torch.int64, device=ints.device)
        for s0 in range(0, k, step):
            ih[s0:s0 + step] = dg.intent_hashes_torch(ints[s0:s0 + step])
        assert (int(ih.sum()) & dg.MASK) == int(g["intent_digest"])
        assert digest_torch(ints[:1 << 20]) == (int(ih[:1 << 20].sum()) & dg.MASK)
        assert dg.positional_torch(ih) == int(g["intent_positional"])
        _check_root_subtrees(g, ih, "intent")
        del ih
        torch.cuda.empty_cache()
        _say("ctx20000x256: intent digests match; order and slices")
        _assert_lectic_increasing(ints, chunk=1 << 24)
        for sl in g["slices"]:
            parts = []
            for s0 in range(0, k, 1 << 26):
                block = ints[s0:s0 + (1 << 26)]
                keep = torch.ones(block.shape[0], dtype=torch.bool, device=ints.device)
                for a in sl["attributes"]:
                    keep &= ((block[:, a >> 6] >> (a & 63)) & 1) != 0
                parts.append(block[keep].cpu().numpy().view(np.uint64))
            sel = np.concatenate(parts)
            assert sel.shape[0] == sl["n_concepts"], sl["attributes"]
            assert hashlib.sha256(np.ascontiguousarray(sel, dtype="<u8").tobytes()).hexdigest() == sl["intents_sha256"]
        del ints, res, block, keep
        torch.cuda.empty_cache()
        # extents, 2^22 rows (10.5 GB) at a time
        page = 1 << 22
        buf = torch.empty((page, 313), dtype=torch.int64, device="cuda")
        eh = torch.empty(k, dtype=torch.int64, device="cuda")
        _say("ctx20000x256: paging extents")
        for first in range(0, k, page):
            cnt = min(page, k - first)
            ctx.write_range(first, extents=buf[:cnt])
            eh[first:first + cnt] = dg.extent_hashes_torch(buf[:cnt])
            if (first // page) % 32 == 0:
                _say("ctx20000x256: extents of rows %d.. hashed" % first)
        assert (int(eh.sum()) & dg.MASK) == int(g["extent_digest"])
        assert dg.positional_torch(eh) == int(g["extent_positional"])
        _check_root_subtrees(g, eh, "extent")
    finally:
        ctx.close()


def _planted(seed, n, m, density, blocks):
    """A random context with `blocks` planted all-ones rectangles (rows and
    columns drawn at random), so that some parents are large and deep."""
    cells = synth.random_context(seed, n, m, density)
    rng = np.random.default_rng(seed + 1)
    for _ in range(blocks):
        r = rng.choice(n, max(1, n // 6), replace=False)
        c = rng.choice(m, max(1, m // 10), replace=False)
        cells[np.ix_(r, c)] = True
    return cells


SWEEP = [(seed, n, m, d, b)
         for seed, (n, m, d, b) in enumerate([(70, 40, 0.3, 1), (150, 66, 0.2, 2), (300, 127, 0.08, 3),
                                               (513, 129, 0.06, 2), (1000, 200, 0.03, 4), (2049, 64, 0.1, 2),
                                               (4100, 90, 0.04, 3), (700, 300, 0.02, 5), (260, 450, 0.015, 4),
                                               (90, 700, 0.01, 2), (5000, 33, 0.15, 1), (129, 257, 0.05, 3)],
                                              start=900)]


@pytest.mark.parametrize("seed,n,m,d,b", SWEEP)
def test_random_shapes_with_planted_blocks(seed, n, m, d, b):
    # shapes on and off word boundaries, densities from 1% to 30%, planted
    # blocks that make large parents (mid and huge classes) and long chains
    assert_parity(_planted(seed, n, m, d, b))


@pytest.mark.parametrize("seed,n,m,d,b", SWEEP)
def test_random_shapes_with_planted_blocks_from_minimal_buffers(seed, n, m, d, b):
    # the same shapes with every buffer starting at its minimum: the store,
    # the record buffers and the huge tests grow level by level, and levels
    # whose records overflowed are redone
    res = assert_parity(_planted(seed, n, m, d, b), flags=fca.FCBO_TINY_BUFFERS)
    assert res.stats["level_redos"] >= 1  # the root (70 objects or more) overflows its one record slot


@pytest.mark.parametrize("n,m,d", [(200, 4096, 0.004), (300, 2000, 0.006)])
def test_wide_intents_with_large_parents(n, m, d):
    # more than eight intent words with parents of more than 64 objects (there
    # every such parent takes the chunked huge path)
    cells = _planted(n * 7 + m, n, m, d, 2)
    assert_parity(cells)


@pytest.mark.parametrize("seed,n,m,d,b", [c for c in SWEEP if c[0] in (905, 906, 907, 908, 909, 910)])
def test_paged_and_streamed_output_on_planted_shapes(seed, n, m, d, b):
    # row widths from 33 to 79 extent words and 1 to 11 intent words: the
    # output kernels' tile shapes, fetched in pieces of seeded random sizes
    # (write_range) and streamed to pinned host memory (copy_to_host)
    cells = _planted(seed, n, m, d, b)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, m)
    k = want.n_concepts
    rng = np.random.default_rng(seed)
    ctx = fca.Context(rows, m)
    try:
        assert ctx.count() == k
        got_i = np.zeros_like(want.intents)
        got_e = np.zeros_like(want.extents)
        bi, be = ctx.alloc_outputs(4096, True)
        first = 0
        while first < k:
            cnt = min(int(rng.integers(1, 4097)), k - first)
            ctx.write_range(first, bi[:cnt], be[:cnt])
            got_i[first:first + cnt] = bi[:cnt].cpu().numpy().view(np.uint64)
            got_e[first:first + cnt] = be[:cnt].cpu().numpy().view(np.uint64)
            first += cnt
        assert np.array_equal(got_i, want.intents)
        assert np.array_equal(got_e, want.extents)
        hi = torch.full((k, ctx.wm), -1, dtype=torch.int64).pin_memory()
        he = torch.full((k, ctx.wn), -1, dtype=torch.int64).pin_memory()
        ctx.copy_to_host(0, k, hi, he, staging_rows=int(rng.integers(100, 3000)))
        assert np.array_equal(hi.numpy().view(np.uint64), want.intents)
        assert np.array_equal(he.numpy().view(np.uint64), want.extents)
    finally:
        ctx.close()


def test_two_contexts_enumerate_at_once_from_two_host_threads():
    # Contexts share no state (the static scratch of the allocation-free entry
    # point aside): two of them, each on a stream of its own, enumerating at
    # the same time from two host threads (ctypes releases the GIL in the
    # library's calls) give the oracle's results, three rounds over
    import threading

    cases = []
    for name in ("ctx2000x64", "ctx10000x128"):
        n, m, _ = synth.CONFIGS[name]
        rows = synth.make_config(name)
        cases.append((name, rows, m, oracle.cbo(rows, m)))
    for rnd in range(3):
        results, errors = {}, []

        def work(name, rows, m):
            try:
                s = torch.cuda.Stream()
                with torch.cuda.stream(s):
                    ctx = fca.Context(rows, m, stream=s)
                    try:
                        res = ctx.enumerate(extents=True)
                        s.synchronize()
                        results[name] = (res.n_concepts, res.intents.cpu().numpy().view(np.uint64),
                                         res.extents.cpu().numpy().view(np.uint64), res.stats["closure_tests"])
                    finally:
                        ctx.close()
            except BaseException as e:  # handed to the main thread
                errors.append((name, e))

        threads = [threading.Thread(target=work, args=(name, rows, m)) for name, rows, m, _ in cases]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), rnd
        assert not errors, errors
        for name, _, _, want in cases:
            k, ints, exts, tests = results[name]
            assert k == want.n_concepts, (rnd, name)
            assert np.array_equal(ints, want.intents), (rnd, name)
            assert np.array_equal(exts, want.extents), (rnd, name)
            assert tests == want.tests, (rnd, name)
