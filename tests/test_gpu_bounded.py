"""GPU parity of the bounded-memory enumeration (fcbo_enumerate_bounded).

Sibling subtrees of the CbO tree are enumerated in batches and the output
handed to a sink piece by piece; the concatenated pieces must equal the
oracle's sorted concept list exactly (intents and extents), with the same
counts, per-level numbers and byte-model inputs.  The batch path is forced on
small contexts with the one-subtree-per-batch and split-root-children hooks and
with a memory limit below what one batch would need; the full-size workloads
run under a limit far below their unbounded footprint and are checked against
the stored oracle values.
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


class Collect:
    """Sink that copies every piece to the host and checks that the pieces
    arrive in order and cover the positions once."""

    def __init__(self):
        self.ints, self.exts, self.next = [], [], 0
        self.pieces = 0
        self.counts = []

    def __call__(self, first, ints, exts):
        assert first == self.next
        count = ints.shape[0] if ints is not None else exts.shape[0]
        if ints is not None:
            self.ints.append(ints.cpu().numpy().view(np.uint64).copy())
        if exts is not None:
            self.exts.append(exts.cpu().numpy().view(np.uint64).copy())
        self.next += count
        self.pieces += 1
        self.counts.append(count)

    def intents(self):
        return np.concatenate(self.ints) if self.ints else None

    def extents(self):
        return np.concatenate(self.exts) if self.exts else None


def run_bounded(rows, m, piece_rows, limit=0, flags=0, intents=True, extents=True, ctx_flags=0):
    ctx = fca.Context(rows, m, flags=ctx_flags)
    try:
        if limit:
            ctx.set_memory_limit(limit)
        sink = Collect()
        k, st = ctx.enumerate_bounded(sink, piece_rows=piece_rows, intents=intents, extents=extents, flags=flags)
        conc, tests = ctx.level_counts()
        return k, st, sink, conc, tests
    finally:
        ctx.close()


def assert_matches_oracle(cells, piece_rows, limit=0, flags=0, ctx_flags=0):
    cells = np.asarray(cells, dtype=bool)
    rows = synth.pack_rows(cells)
    m = cells.shape[1]
    want = oracle.cbo(rows, m, keep_extents=True)
    k, st, sink, conc, tests = run_bounded(rows, m, piece_rows, limit, flags, ctx_flags=ctx_flags)
    assert k == want.n_concepts == sink.next
    assert np.array_equal(sink.intents(), want.intents)
    assert np.array_equal(sink.extents(), want.extents)
    assert st["closure_tests"] == want.tests
    assert st["item_pairs"] == want.pairs
    assert st["sum_child_objects"] == want.sum_c
    assert st["local_parent_objects"] + st["medium_parent_objects"] == want.sum_rl_objs
    assert st["big_parents"] == want.col_parents
    assert st["big_nonzero_words"] == want.col_nzw
    assert st["big_child_objects"] == want.col_child_objs
    assert st["model_bytes"] == oracle.model_bytes(want)
    assert [int(x) for x in conc] == [int(x) for x in want.level_concepts]
    assert [int(x) for x in tests] == [int(x) for x in want.level_tests]
    assert sink.pieces >= -(-k // piece_rows)
    assert all(c <= piece_rows for c in sink.counts)
    return k, st, want


# --- small contexts, batches forced by the hooks -----------------------------------------

ONE = fca.FCBO_ONE_SUBTREE_PER_BATCH
SPLIT = fca.FCBO_SPLIT_ROOT_CHILDREN


@pytest.mark.parametrize("name", ["staircase4.txt", "two_blocks4.txt"])
@pytest.mark.parametrize("flags", [ONE, SPLIT, ONE | SPLIT])
def test_hand_derived_examples(name, flags):
    cells, _, info = read_fixture(name)
    k, st, _ = assert_matches_oracle(cells, piece_rows=3, flags=flags)
    assert k == info["concepts"]


@pytest.mark.parametrize("name,piece", [("ctx64x16", 7), ("ctx2000x64", 1000), ("ctx10000x128", 4099)])
def test_seeded_contexts_one_subtree_per_batch(name, piece):
    cells = synth.make_config(name, packed=False)
    k, st, want = assert_matches_oracle(cells, piece_rows=piece, flags=ONE)
    # one batch per child of the root (level 1 of the CbO tree)
    assert st["batches"] == int(want.level_concepts[1])
    assert st["batch_retries"] == 0 and st["batch_splits"] == 0
    # the hook withholds the seeds' classes: a seed of more than 64 objects
    # makes its batch's first level run again with the mid / huge kernels
    if name != "ctx64x16":  # there every concept has at most 64 objects
        assert st["level_redos"] >= 1


@pytest.mark.parametrize("name,piece", [("ctx64x16", 5), ("ctx2000x64", 999), ("ctx10000x128", 1 << 20)])
@pytest.mark.parametrize("one", [False, True])
def test_seeded_contexts_root_children_split(name, piece, one):
    # every root child's row goes out on its own, its children's subtrees
    # follow as batches of the next level
    cells = synth.make_config(name, packed=False)
    k, st, want = assert_matches_oracle(cells, piece_rows=piece, flags=SPLIT | (ONE if one else 0))
    assert st["batch_splits"] == int(want.level_concepts[1])
    if one:
        assert st["batches"] == int(want.level_concepts[2])


@pytest.mark.parametrize("name", ["ctx2000x64", "ctx10000x128"])
def test_tiny_buffers_one_subtree_per_batch(name):
    # every buffer starts at its minimum size: growth and the level redo run
    # inside the batches
    cells = synth.make_config(name, packed=False)
    assert_matches_oracle(cells, piece_rows=2048, flags=ONE, ctx_flags=fca.FCBO_TINY_BUFFERS)


def test_all_ones_and_all_zero():
    # all-ones: the root holds every attribute and is the only concept (no batch)
    k, st, _ = assert_matches_oracle(synth.all_ones(70, 130), piece_rows=4, flags=SPLIT)
    assert k == 1 and st["batches"] == 0 and st["batch_splits"] == 0
    # all-zero: the root (all objects, no attribute) and the bottom (no object,
    # every attribute), the root's only child
    k, st, _ = assert_matches_oracle(synth.all_zero(70, 5), piece_rows=4)
    assert k == 2 and st["batches"] == 1
    k, st, _ = assert_matches_oracle(synth.all_zero(70, 5), piece_rows=4, flags=SPLIT)
    assert k == 2 and st["batches"] == 0 and st["batch_splits"] == 1


@pytest.mark.parametrize("k", [2, 5, 64, 65])
def test_diagonal(k):
    # the diagonal context of size k: k + 2 concepts, one batch per atom
    k_, st, _ = assert_matches_oracle(synth.diagonal(k), piece_rows=2, flags=ONE)
    assert k_ == k + 2
    assert_matches_oracle(synth.diagonal(k), piece_rows=1, flags=SPLIT)


# --- the memory limit decides the batches ------------------------------------------------

def _unbounded_peak(rows, m, ctx_flags=0):
    ctx = fca.Context(rows, m, flags=ctx_flags)
    try:
        sink = Collect()
        k, st = ctx.enumerate_bounded(sink, piece_rows=1 << 16, intents=True, extents=False)
        return k, st
    finally:
        ctx.close()


def test_memory_limit_splits_the_root_children():
    cells = synth.make_config("ctx10000x128", packed=False)
    rows = synth.pack_rows(cells)
    k0, st0 = _unbounded_peak(rows, 128, fca.FCBO_TINY_BUFFERS)
    assert st0["batches"] == 1 and st0["batch_retries"] == 0
    # a third of the one-batch footprint: the library must split, retry and still
    # deliver every concept in order
    limit = st0["peak_device_bytes"] // 3
    k, st, _ = assert_matches_oracle(cells, piece_rows=1 << 14, limit=limit, ctx_flags=fca.FCBO_TINY_BUFFERS)
    assert k == k0
    assert st["batches"] >= 2
    assert st["batch_retries"] >= 1
    assert st["peak_device_bytes"] <= limit


def test_limit_below_the_root_fails_cleanly():
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    ctx = fca.Context(rows, 64, flags=fca.FCBO_TINY_BUFFERS)
    try:
        ctx.set_memory_limit(4 << 10)  # 4 KiB: not even the root's extent list fits
        with pytest.raises(fca.FcboError) as e:
            ctx.enumerate_bounded(Collect(), piece_rows=1024)
        assert e.value.code == fca.FCBO_ERR_OUT_OF_MEMORY
        # nothing of the failed call survives; the context still works
        with pytest.raises(fca.FcboError):
            ctx.level_counts()
        ctx.set_memory_limit(0)
        want = oracle.cbo(rows, 64, keep_extents=False)
        res = ctx.enumerate(extents=False)
        assert res.n_concepts == want.n_concepts
        assert np.array_equal(res.intents.cpu().numpy().view(np.uint64), want.intents)
    finally:
        ctx.close()


# --- sinks ---------------------------------------------------------------------------------

def test_count_only_and_outputs_one_at_a_time():
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 64, keep_extents=True)
    ctx = fca.Context(rows, 64)
    try:
        calls = []
        k, st = ctx.enumerate_bounded(lambda *a: calls.append(a), intents=False, extents=False,
                                      flags=fca.FCBO_ONE_SUBTREE_PER_BATCH)
        assert k == want.n_concepts and not calls
        assert st["closure_tests"] == want.tests and st["output_bytes"] == 0
        sink = Collect()
        k, st = ctx.enumerate_bounded(sink, piece_rows=777, intents=False, extents=True)
        assert np.array_equal(sink.extents(), want.extents) and sink.intents() is None
        sink = Collect()
        k, st = ctx.enumerate_bounded(sink, piece_rows=777, intents=True, extents=False,
                                      flags=fca.FCBO_ONE_SUBTREE_PER_BATCH)
        assert np.array_equal(sink.intents(), want.intents) and sink.extents() is None
        assert st["output_bytes"] == k * 8
    finally:
        ctx.close()


def test_sink_stops_and_sink_errors_propagate():
    cells = synth.make_config("ctx2000x64", packed=False)
    rows = synth.pack_rows(cells)
    ctx = fca.Context(rows, 64)
    try:
        seen = []

        def stop_after_two(first, ints, exts):
            seen.append(first)
            return len(seen) >= 2

        with pytest.raises(fca.FcboError) as e:
            ctx.enumerate_bounded(stop_after_two, piece_rows=1000, extents=False)
        assert e.value.code == fca.FCBO_ERR_STOPPED
        assert seen == [0, 1]  # the root's row on its own, then the first batch
        # no result and no level counts are left behind
        buf = torch.empty((10, 1), dtype=torch.int64, device="cuda")
        with pytest.raises(fca.FcboError):
            ctx.write_range(0, intents=buf)
        with pytest.raises(fca.FcboError):
            ctx.level_counts()

        def boom(first, ints, exts):
            raise KeyError("from the sink")

        with pytest.raises(KeyError):
            ctx.enumerate_bounded(boom, piece_rows=1000, extents=False)
        # the context is still usable
        want = oracle.cbo(rows, 64, keep_extents=False)
        sink = Collect()
        k, _ = ctx.enumerate_bounded(sink, piece_rows=1 << 20, extents=False)
        assert k == want.n_concepts and np.array_equal(sink.intents(), want.intents)
    finally:
        ctx.close()


def test_bounded_then_normal_enumeration_on_one_context():
    cells = synth.make_config("ctx10000x128", packed=False)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, 128, keep_extents=True)
    ctx = fca.Context(rows, 128)
    try:
        sink = Collect()
        ctx.enumerate_bounded(sink, piece_rows=5000, flags=fca.FCBO_ONE_SUBTREE_PER_BATCH)
        assert np.array_equal(sink.intents(), want.intents)
        res = ctx.enumerate(extents=True)
        assert np.array_equal(res.intents.cpu().numpy().view(np.uint64), want.intents)
        assert np.array_equal(res.extents.cpu().numpy().view(np.uint64), want.extents)
    finally:
        ctx.close()


# --- the full-size workloads under a memory limit ----------------------------------------

def _say(msg):
    print("[bounded] %s" % msg, flush=True)


class HashSink:
    """Hashes every piece on the device: per-position intent and extent hashes
    into preallocated device arrays, and lexicographic order across pieces."""

    def __init__(self, k, device="cuda", extents=True):
        self.ih = torch.empty(k, dtype=torch.int64, device=device)
        self.eh = torch.empty(k, dtype=torch.int64, device=device) if extents else None
        self.next = 0
        self.last = None
        self.k = k
        self.pieces = 0

    def __call__(self, first, ints, exts):
        assert first == self.next
        cnt = ints.shape[0]
        assert first + cnt <= self.k
        self.ih[first:first + cnt] = dg.intent_hashes_torch(ints)
        if self.eh is not None:
            self.eh[first:first + cnt] = dg.extent_hashes_torch(exts)
        rows = ints if self.last is None else torch.cat([self.last, ints])
        _lectic_increasing(rows)
        self.last = ints[-1:].clone()
        self.next += cnt
        self.pieces += 1
        if self.pieces % 64 == 0:
            _say("rows %d.. hashed" % first)
        torch.cuda.current_stream().synchronize()  # done with the piece buffers


def _lectic_increasing(ints):
    if ints.shape[0] < 2:
        return
    a, b = ints[:-1], ints[1:]
    x = a ^ b
    nz = x != 0
    assert bool(nz.any(dim=1).all()), "equal neighbouring intents"
    first = nz.int().argmax(dim=1)
    xw = x.gather(1, first[:, None]).squeeze(1)
    bw = b.gather(1, first[:, None]).squeeze(1)
    assert bool(((bw & (xw & (-xw))) != 0).all()), "rows out of lexicographic order"


def _check_root_subtrees(g, hashes, which):
    start = 1
    lo = 2 if which == "intent" else 4
    for attr, size, *sums in g["root_children"]:
        part = hashes[start:start + size]
        assert (int(part.sum()) & dg.MASK) == int(sums[lo - 2]), (which, attr)
        assert dg.positional_torch(part) == int(sums[lo - 1]), (which, attr)
        start += size
    assert start == hashes.shape[0]


def test_full_ctx50000x400_bounded_against_stored_oracle():
    release_device_cache()
    path = os.path.join(GOLDEN, "ctx50000x400.json")
    if not os.path.exists(path):
        pytest.skip("stored oracle values not generated")
    g = json.load(open(path))
    rows = synth.make_config("ctx50000x400")
    assert synth.rows_sha256(rows) == g["rows_sha256"]
    ctx = fca.Context(rows, 400)
    try:
        limit = 256 << 20  # a quarter of a GiB for every enumeration buffer
        ctx.set_memory_limit(limit)
        k = g["n_concepts"]
        ints_all = torch.empty((k, 7), dtype=torch.int64, device="cuda")
        hs = HashSink(k)

        def sink(first, ints, exts):
            ints_all[first:first + ints.shape[0]] = ints
            hs(first, ints, exts)

        _say("ctx50000x400 under %d MiB" % (limit >> 20))
        k2, st = ctx.enumerate_bounded(sink, piece_rows=1 << 18)
        assert k2 == k and hs.next == k
        assert st["peak_device_bytes"] <= limit and st["batches"] >= 2
        conc, tests = ctx.level_counts()
        assert st["closure_tests"] == g["closure_tests"]
        assert st["item_pairs"] == g["item_pairs"]
        assert st["sum_child_objects"] == g["sum_c"]
        assert st["model_bytes"] == g["model_bytes"]
        assert [int(x) for x in conc] == g["level_concepts"]
        assert [int(x) for x in tests] == g["level_tests"]
        ints = ints_all.cpu().numpy().view(np.uint64)
        assert hashlib.sha256(np.ascontiguousarray(ints, dtype="<u8").tobytes()).hexdigest() == g["intents_sha256"]
        ehs = hs.eh.cpu().numpy().view(np.uint64)
        assert hashlib.sha256(np.ascontiguousarray(ehs, dtype="<u8").tobytes()).hexdigest() == g["extent_hashes_sha256"]
        assert dg.positional_torch(hs.ih) == int(g["intent_positional"])
        assert dg.positional_torch(hs.eh) == int(g["extent_positional"])
        _say("ctx50000x400: %d batches, %d retries, peak %.1f MiB"
             % (st["batches"], st["batch_retries"], st["peak_device_bytes"] / 2**20))
    finally:
        ctx.close()


def test_full_ctx20000x256_bounded_against_store_free_oracle():
    # 1.41e9 concepts whose store alone takes some 150 GB, enumerated with
    # 24 GiB for every enumeration buffer; intents and all 3.5 TB of extents
    # pass through 2^21-row pieces and are hashed on the device.
    release_device_cache()
    path = os.path.join(GOLDEN, "ctx20000x256.json")
    if not os.path.exists(path):
        pytest.skip("stored oracle values not generated")
    g = json.load(open(path))
    rows = synth.make_config("ctx20000x256")
    assert synth.rows_sha256(rows) == g["rows_sha256"]
    ctx = fca.Context(rows, 256)
    try:
        limit = 24 << 30
        ctx.set_memory_limit(limit)
        k = g["n_concepts"]
        hs = HashSink(k)
        _say("ctx20000x256 under %d GiB" % (limit >> 30))
        k2, st = ctx.enumerate_bounded(hs, piece_rows=1 << 21)
        assert k2 == k and hs.next == k
        assert st["peak_device_bytes"] <= limit and st["batches"] >= 2
        conc, tests = ctx.level_counts()
        assert st["closure_tests"] == g["closure_tests"]
        assert st["item_pairs"] == g["item_pairs"]
        assert st["sum_child_objects"] == g["sum_c"]
        assert [int(x) for x in conc] == g["level_concepts"]
        assert [int(x) for x in tests] == g["level_tests"]
        assert (int(hs.ih.sum()) & dg.MASK) == int(g["intent_digest"])
        assert dg.positional_torch(hs.ih) == int(g["intent_positional"])
        assert (int(hs.eh.sum()) & dg.MASK) == int(g["extent_digest"])
        assert dg.positional_torch(hs.eh) == int(g["extent_positional"])
        _check_root_subtrees(g, hs.ih, "intent")
        _check_root_subtrees(g, hs.eh, "extent")
        _say("ctx20000x256: %d batches, %d retries, peak %.2f GiB, %.1f s"
             % (st["batches"], st["batch_retries"], st["peak_device_bytes"] / 2**30, st["enumerate_ms"] / 1e3))
    finally:
        ctx.close()
        hs = None
        release_device_cache()


from tests.test_gpu_parity import SWEEP, _planted  # noqa: E402


@pytest.mark.parametrize("seed,n,m,d,b", SWEEP[:6])
def test_random_shapes_with_planted_blocks_in_batches(seed, n, m, d, b):
    # every batch one subtree (the hook), pieces of a few hundred rows
    assert_matches_oracle(_planted(seed, n, m, d, b), piece_rows=333, flags=ONE)


@pytest.mark.parametrize("seed,n,m,d,b", SWEEP[6:])
def test_random_shapes_with_planted_blocks_split_below_the_root(seed, n, m, d, b):
    # every root child split one level down (the hook), so the batches hold
    # grandchildren of the root; pieces of a thousand rows
    k, st, want = assert_matches_oracle(_planted(seed, n, m, d, b), piece_rows=1000, flags=SPLIT)
    assert st["batch_splits"] == int(want.level_concepts[1])
