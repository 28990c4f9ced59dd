"""The allocation-free entry point against fcbo_enumerate, through the C ABI.

fcbo_enumerate_static carves every device buffer from the library's static
scratch.  Two calls in a row on one device (the second on a smaller context,
so stale scratch contents of the first would show), each compared row for row
with fcbo_enumerate on the same input and with the CPU oracle.
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


def _static_call(rows_dev, n, m, capacity, extents=True):
    wm, wn = (m + 63) // 64, (n + 63) // 64
    ints = torch.full((max(capacity, 1), wm), -1, dtype=torch.int64, device="cuda")
    exts = torch.full((max(capacity, 1), wn), -1, dtype=torch.int64, device="cuda") if extents else None
    stream = torch.cuda.current_stream().cuda_stream
    rc, k, st = fca.fcbo_enumerate_static(rows_dev.data_ptr(), n, m, rows_dev.shape[1], fca.FCBO_ROWS_ON_DEVICE,
                                          stream, ints.data_ptr(), exts.data_ptr() if extents else 0, capacity)
    torch.cuda.synchronize()
    return rc, k, st, ints, exts


def test_static_entry_matches_enumerate_on_two_calls_second_smaller():
    for name in ("ctx2000x64", "ctx64x16"):
        n, m, _ = synth.CONFIGS[name]
        rows = synth.make_config(name)
        ctx = fca.Context(rows, m)
        try:
            ref = ctx.enumerate(extents=True)
            torch.cuda.synchronize()
        finally:
            ctx.close()
        k = ref.n_concepts
        rows_dev = torch.from_numpy(rows.view(np.int64)).cuda()
        rc, kk, st, ints, exts = _static_call(rows_dev, n, m, k)
        assert rc == fca.FCBO_OK and kk == k, name
        assert torch.equal(ints, ref.intents), name
        assert torch.equal(exts, ref.extents), name
        for key in ("closure_tests", "item_pairs", "n_levels", "sum_child_objects", "model_bytes"):
            assert getattr(st, key) == ref.stats[key], (name, key)
        want = oracle.cbo(rows, m)
        assert np.array_equal(ints.cpu().numpy().view(np.uint64), want.intents)
        assert np.array_equal(exts.cpu().numpy().view(np.uint64), want.extents)


def test_static_entry_capacity_and_scratch_errors():
    n, m, _ = synth.CONFIGS["ctx64x16"]
    rows = synth.make_config("ctx64x16")
    rows_dev = torch.from_numpy(rows.view(np.int64)).cuda()
    want = oracle.cbo(rows, m)
    rc, kk, _, ints, exts = _static_call(rows_dev, n, m, want.n_concepts - 1)
    assert rc == fca.FCBO_ERR_CAPACITY and kk == want.n_concepts
    assert bool((ints == -1).all()) and bool((exts == -1).all())
    # intents only, host rows
    ints = torch.full((want.n_concepts, 1), -1, dtype=torch.int64, device="cuda")
    rc, kk, _ = fca.fcbo_enumerate_static(rows.ctypes.data, n, m, 1, 0, torch.cuda.current_stream().cuda_stream,
                                          ints.data_ptr(), 0, want.n_concepts)
    torch.cuda.synchronize()
    assert rc == fca.FCBO_OK and kk == want.n_concepts
    assert np.array_equal(ints.cpu().numpy().view(np.uint64), want.intents)
    # an enumeration that outgrows the scratch: 2^20 concepts (their intents,
    # cursors, offsets and extent lists alone take more than 64 MiB)
    cells = synth.pad_with_full(synth.contranominal(20), extra_objects=2, extra_attrs=2)
    big = synth.pack_rows(cells)
    big_dev = torch.from_numpy(big.view(np.int64)).cuda()
    rc, kk, _, _, _ = _static_call(big_dev, cells.shape[0], cells.shape[1], 0, extents=False)
    assert rc == fca.FCBO_ERR_SCRATCH


from tests.test_gpu_parity import SWEEP, _planted  # noqa: E402


@pytest.mark.parametrize("seed,n,m,d,b", SWEEP)
def test_static_entry_on_random_shapes_with_planted_blocks(seed, n, m, d, b):
    # shapes on and off word boundaries (up to eleven intent words), planted
    # blocks that make mid and huge parents: every level kernel and buffer
    # growth, all of it carved from the static scratch, against the oracle
    cells = _planted(seed, n, m, d, b)
    rows = synth.pack_rows(cells)
    want = oracle.cbo(rows, m)
    rows_dev = torch.from_numpy(rows.view(np.int64)).cuda()
    rc, k, st, ints, exts = _static_call(rows_dev, n, m, want.n_concepts)
    assert rc == fca.FCBO_OK and k == want.n_concepts
    assert np.array_equal(ints.cpu().numpy().view(np.uint64), want.intents)
    assert np.array_equal(exts.cpu().numpy().view(np.uint64), want.extents)
    assert st.closure_tests == want.tests and st.item_pairs == want.pairs
    assert st.sum_child_objects == want.sum_c
