"""bench.py's command-line contract and its byte model (CPU only)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_output_byte_model_counts_reads_and_writes():
    # K = 3 concepts, N = 130 objects (3 extent words), M = 70 attributes (2
    # intent words), 5 objects in the children's lists.  The intent pass reads
    # a permutation entry (4) and an intent (16) per concept and writes the
    # intent (16); the extent pass reads the permutation entry again (4), the
    # list bounds (16) and every list entry (4 each: the root's 130 objects and
    # the children's 5), and writes 24 bytes of extent per concept.
    st = {"sum_child_objects": 5}
    intents_only = 3 * (4 + 16) + 3 * 16
    assert bench.kernel_bytes("output", st, wm=2, wn=3, n=130, k=3, extents=False) == intents_only
    got = bench.kernel_bytes("output", st, wm=2, wn=3, n=130, k=3, extents=True)
    assert got == intents_only + 3 * (4 + 16) + (130 + 5) * 4 + 3 * 24
