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


def test_traffic_records_are_kept_only_for_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    # A counter summary holds one record per kernel class with the hash of the
    # device sources it was measured on; a record whose hash differs from the
    # sources in the tree is dropped, so a changed kernel reports no traffic.
    csrc = tmp_path / "closed_set_enumeration_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "fcbo_device.h").write_bytes(b"device header\n")
    (csrc / "fcbo.hip").write_bytes(b"host source\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.source_sha256()
    (tmp_path / "profiles" / "w_traffic.md").write_text(
        "# summary\n"
        "traffic-record: class=output source_sha256=%s fetch=1 write=2\n"
        "traffic-record: class=level_loop source_sha256=%s fetch=3 write=4\n"
        "not a record: class=other\n" % (sha, "0" * 64))
    got = bench.profile_records("w")
    assert list(got) == ["output"]
    assert got["output"]["fetch"] == "1" and got["output"]["write"] == "2"
    assert bench.profile_records("missing") == {}
    (csrc / "fcbo.hip").write_bytes(b"host source, edited\n")
    assert bench.profile_records("w") == {}


def test_task_pool_schedule_beyond_512_attributes_is_refused_before_any_device_work(monkeypatch):
    import synth

    monkeypatch.setitem(synth.CONFIGS, "wide", (10, 513, None))
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "wide", "--schedule", "pool", "--no-cpu"])
    try:
        bench.main()
    except SystemExit as e:
        assert e.code == 2
    else:
        raise AssertionError("bench.main() accepted 513 attributes with the task pool")


def _write_counters(path, rows):
    import csv

    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_sq_summary_issue_share_and_valu_counts(tmp_path, capsys):
    # One dispatch of 1 ms issuing 6.144e8 VALU wave-instructions: at four
    # cycles each that is the whole issue capacity of 256 CUs x 4 SIMDs at
    # 2.4 GHz (share 1.0); a second kernel at a quarter of it over 2 ms.
    a, b = tmp_path / "a.csv", tmp_path / "b.csv"
    k1, k2 = "void fcbo::k_local_test<7>(fcbo::LevelArgs)", "fcbo::k_scan_up(...)"
    _write_counters(a, [
        {"Dispatch_Id": 1, "Kernel_Name": k1, "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": 6.144e8,
         "Start_Timestamp": 0, "End_Timestamp": 1_000_000},
        {"Dispatch_Id": 2, "Kernel_Name": k2, "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": 3.072e8,
         "Start_Timestamp": 0, "End_Timestamp": 2_000_000},
    ])
    _write_counters(b, [
        {"Dispatch_Id": 1, "Kernel_Name": k1, "Counter_Name": "SQ_WAIT_ANY", "Counter_Value": 5,
         "Start_Timestamp": 0, "End_Timestamp": 1_000_000},
    ])
    issue, valu = bench.rocprof_sq(str(a), str(b))
    capsys.readouterr()
    assert abs(issue["k_local_test<7>"] - 1.0) < 1e-9
    assert abs(issue["k_scan_up"] - 0.25) < 1e-9
    assert valu == {"k_local_test<7>": 6.144e8, "k_scan_up": 3.072e8}
    # the issue-rate peak the bench divides by: 614.4 G wave-instructions a second
    assert abs(bench.VALU_ISSUE_PEAK_G - 614.4) < 1e-9


def test_kernel_trace_gaps_of_the_last_level_loop(tmp_path, capsys):
    # Two enumerations; only the second one's level loop (from its k_root_init to
    # its first k_subtree_size) is read.  Its kernels, in us from its start:
    #   root [0, 100) s0, test [100, 400) s0, mid [420, 500) s1, write [450, 600)
    #   s0 (overlapping mid), then the ordering kernel at 630.  Some kernel runs
    #   in [0, 400) and [420, 600): 580 of a 630 us span; the gaps are 20 us
    #   (s0 test -> s1 mid, across streams) and 30 us (write -> ordering).
    head = '"Kind","Dispatch_Id","Kernel_Name","Stream_Id","Start_Timestamp","End_Timestamp"\n'
    us = 1000
    t = 50_000 * us
    rows = [("fcbo::k_root_init(x)", 0, 0, 50 * us), ("fcbo::k_subtree_size(x)", 0, 60 * us, 70 * us),
            ("fcbo::k_root_init(x)", 0, t, t + 100 * us),
            ("void fcbo::k_local_test<7>(x)", 0, t + 100 * us, t + 400 * us),
            ("void fcbo::k_mid_test<7>(x)", 1, t + 420 * us, t + 500 * us),
            ("void fcbo::k_local_write<7>(x)", 0, t + 450 * us, t + 600 * us),
            ("fcbo::k_subtree_size(x)", 0, t + 630 * us, t + 700 * us)]
    p = tmp_path / "trace_kernel_trace.csv"
    p.write_text(head + "".join('"KERNEL_DISPATCH",%d,"%s",%d,%d,%d\n' % (i, n, q, s, e)
                                for i, (n, q, s, e) in enumerate(rows)))
    bench.rocprof_gaps(str(p))
    out = capsys.readouterr().out
    assert "| 630.0 | 580.0 | 50.0 | 2 | 1 | 20.0 |" in out
    gaps = [ln for ln in out.splitlines() if ln.startswith("| 600.0 |") or ln.startswith("| 400.0 |")]
    # longest first: 30 us after the write, then 20 us across streams
    assert gaps == ["| 600.0 | 30.0 | `k_local_write<7>` (0) | `k_subtree_size` (0) |",
                    "| 400.0 | 20.0 | `k_local_test<7>` (0) | `k_mid_test<7>` (1) |"]
