"""Benchmark: concept enumeration throughput on one MI355X.

One step = one full call of fcbo_enumerate on a seeded context: the root, every
level of closure tests and child writes, the output ordering and the ordered
intents (plus, when they fit in device memory, the extent bitmaps) written to
preallocated device buffers.  The context is resident in HBM before timing
starts.  The default workload is the 50,000 x 400 context.

    python bench.py [--gpus 1] [--steps 5] [--warmup 1] [--workload ctx50000x400]

Prints one JSON line.  `value` is concepts per second; beside it:
  * closure tests per second;
  * `roofline`: the dominant kernel class (the output writer), its algorithmic
    bytes over its launch time, measured live on every timed step with HIP
    events on the library's stream, against the 8 TB/s HBM peak;
  * `closure_roofline`: the level loop (root to last level: closure tests,
    scans, child writes, the per-level host wait), the library's algorithmic
    byte count `model_bytes` over its measured time, and (`alu`) its VALU
    wave-instructions per step from the committed counter pass over the same
    time, against the chip's issue rate (the bound these kernels meet);
  * `hbm_probe`: a device copy and a fill timed in the same process, the
    achievable bandwidth on this machine, and a fill of the extent buffer itself
    (the store rate a destination of that size allows);
  * `cover_edges`: the lattice's cover edges of the same result
    (fcbo_cover_edges), timed once after the steps;
  * `host_stream`: the first rows of the ordered output streamed to pinned
    host memory through two device staging buffers (fcbo_copy_to_host), a
    PCIe-inclusive rate, never the headline value;
  * `task_pool`: the same step with the task-pool schedule (FCBO_TASK_POOL:
    the level loop expands only parents with more than 16 objects, one
    wavefront enumerates each smaller concept's subtree depth-first), timed
    over its own steps into the same buffers;
  * `bounded`: the same enumeration in bounded device memory
    (fcbo_enumerate_bounded under fcbo_set_memory_limit, by default a quarter
    of what the unbounded step held), the whole output (intents and extent
    bitmaps) handed to a no-op sink piece by piece;
  * `cpu_baseline`: the store-free CPU oracle over the whole workload on one
    pinned host core, run before the GPU is touched; `cpu_baseline_all_cores`
    the same search split over the host cores.

The per-class breakdown (`kernel_ms`) comes from one extra, untimed step with
an event pair around every kernel class (recording them costs about 0.6 ms a
step on the 50,000 x 400 context, so the timed steps run without).  Parts of a
level run on the library's side streams, so the classes that overlap there
(mid and huge tests, the writers) include waiting and add up to more than the
level loop; the output kernels run alone.

    python bench.py --rocprof-summary <kernel_stats.csv or counter_collection.csv> ...

turns rocprofv3 CSV files into the tables kept under profiles/ (see there).
"""

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
VALU_ISSUE_PEAK_G = 256 * 4 * 2.4 / 4  # wave64 VALU instructions per ns: 256 CUs x 4 SIMDs at 2.4 GHz, 4 cycles each
LEVEL_LOOP_KERNELS = ("k_local_test", "k_mid_test", "k_mid_test_wide", "k_huge_tasks", "k_huge_partial",
                      "k_huge_finalize", "k_big_test_list", "k_local_write", "k_mid_write", "k_mid_write_wide",
                      "k_huge_write", "k_big_write_list", "k_scan_up", "k_scan_mid", "k_scan_down", "k_scan_small",
                      "k_root_init", "k_root_and", "k_fill_u64")


def kernel_bytes(cls, st, wm, wn, n, k, extents):
    """Algorithmic bytes one step moves in a kernel class."""
    if cls == "output":
        # intents: permutation entry and intent in, intent out; extents: the
        # permutation entry again, list bounds and the list in, extent row out
        # (every concept's list: the root's N objects plus the children's)
        b = k * (4 + 8 * wm) + k * 8 * wm
        if extents:
            b += k * (4 + 16) + (n + st["sum_child_objects"]) * 4 + k * 8 * wn
        return b
    if cls == "order":
        # subtree sizes: first-child offset, the children's sizes, the size out; positions:
        # offset, own position, the children's sizes in and positions out; inverse: position in,
        # concept index out
        return k * (4 + 4 + 4) + k * (4 + 4 + 4 + 4) + k * (4 + 4)
    return None


def source_sha256():
    """SHA-256 of the device sources (kernels and their launch code)."""
    import hashlib

    h = hashlib.sha256()
    for f in ("closed_set_enumeration_amd/csrc/fcbo_device.h", "closed_set_enumeration_amd/csrc/fcbo.hip"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_records(workload):
    """`traffic-record:` lines of the committed counter summary of a workload, keyed by class,
    kept only while the device sources hash to the value they were taken on."""
    path = os.path.join(ROOT, "profiles", "%s_traffic.md" % workload)
    out = {}
    if not os.path.exists(path):
        return out
    sha = source_sha256()
    with open(path) as f:
        for line in f:
            if not line.startswith("traffic-record:"):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[1:])
            if kv.get("source_sha256") == sha:
                out[kv["class"]] = kv
    return out


def column_streaming_what_if(workload, loop_ms):
    """The bandwidth a column-streaming closure (one read of col[j] at every
    non-zero word of the parent extent per test, the pages' design) would need to
    make the same closure tests in the measured level-loop time.  Not an achieved
    rate: the kernels here read rows once per parent instead."""
    path = os.path.join(ROOT, "tests", "golden", "%s.json" % workload)
    if not os.path.exists(path) or loop_ms <= 0:
        return None
    with open(path) as f:
        g = json.load(f)
    if "sum_nzw" not in g:
        return None
    gbytes = 8.0 * g["sum_nzw"] / 1e9
    return {"column_bytes_GB": round(gbytes, 2), "level_loop_ms": round(loop_ms, 4),
            "required_GBps": round(gbytes / (loop_ms * 1e-3), 1)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_cores():
    try:
        return sorted(os.sched_getaffinity(0))
    except AttributeError:
        return list(range(os.cpu_count() or 1))


def cpu_baselines(rows, m, threads_all, bitmap_tests):
    """The oracle on the host cores, before the GPU is touched.  The store-free
    search (object lists) covers the whole workload: once on one core (the calling
    thread pinned to it, the worker it starts inherits that), once split over
    `threads_all` cores.  The bitmap search runs a bounded depth-first prefix as a
    labelled extra."""
    import oracle

    cores = host_cores()
    info = {"cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity_cores": len(cores)}
    out = {}
    old = None
    try:
        old = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {cores[0]})
    except (AttributeError, OSError):
        old = None
    try:
        t0 = time.perf_counter()
        d = oracle.cbo_digest(rows, m, threads=1)
        wall = time.perf_counter() - t0
    finally:
        if old is not None:
            os.sched_setaffinity(0, old)
    out["one"] = dict(info, **{
        "value": round(d.n_concepts / d.seconds, 1), "unit": "concepts/s",
        "closure_tests_per_s": round(d.tests / d.seconds, 1), "cores": 1, "kind": "oracle",
        "sample": "whole workload: store-free CbO oracle (object-list extents), %d concepts, %d closure tests, "
                  "%.2f s search (%.2f s wall), one pinned core" % (d.n_concepts, d.tests, d.seconds, wall),
        "seconds": round(d.seconds, 3)})
    t0 = time.perf_counter()
    d = oracle.cbo_digest(rows, m, threads=threads_all)
    wall = time.perf_counter() - t0
    out["all"] = dict(info, **{
        "value": round(d.n_concepts / d.seconds, 1), "unit": "concepts/s",
        "closure_tests_per_s": round(d.tests / d.seconds, 1), "cores": d.threads, "kind": "oracle",
        "sample": "whole workload: the same search, subtrees of the root's children over %d threads, "
                  "%.2f s search (%.2f s wall)" % (d.threads, d.seconds, wall),
        "seconds": round(d.seconds, 3)})
    if bitmap_tests > 0:
        r = oracle.cbo(rows, m, keep_extents=False, max_tests=bitmap_tests)
        secs = r.seconds_enum + r.seconds_sort
        out["bitmap"] = {
            "value": round(r.n_concepts / secs, 1), "unit": "concepts/s",
            "closure_tests_per_s": round(r.tests / secs, 1), "cores": 1, "kind": "oracle",
            "sample": "bitmap CbO oracle (column AND per test), depth-first prefix stopped after %d closure "
                      "tests (%d concepts, %.2f s); a prefix, not the whole workload" % (r.tests, r.n_concepts, secs)}
    return out


def hbm_probe(torch, gib):
    """A device-to-device copy and a fill of `gib` GiB, HIP events around each."""
    nel = int(gib * (1 << 30)) // 8
    src = torch.ones(nel, dtype=torch.int64, device="cuda")
    dst = torch.empty_like(src)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(2):  # first pass warms up
        e[0].record()
        dst.copy_(src)
        e[1].record()
        dst.zero_()
        e[2].record()
        torch.cuda.synchronize()
    copy_ms, fill_ms = e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])
    nbytes = nel * 8
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "copy_GBps": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1),
            "fill_GBps": round(nbytes / (fill_ms * 1e-3) / 1e9, 1)}


# --- rocprofv3 CSV summaries ------------------------------------------------------------

def rocprof_summary(paths):
    """Print markdown tables from rocprofv3 CSVs: kernel_stats (name, calls, total,
    average ns) or counter_collection (per kernel: dispatches, counter sums)."""
    import csv

    for path in paths:
        with open(path) as f:
            rows = list(csv.DictReader(f))
        if not rows:
            continue
        print("## %s\n" % os.path.basename(path))
        if "Counter_Name" in rows[0]:
            agg = {}
            for r in rows:
                name = r["Kernel_Name"].split("(")[0]
                key = (name, r["Counter_Name"])
                a = agg.setdefault(key, [0, 0.0, set()])
                a[1] += float(r["Counter_Value"])
                a[2].add(r.get("Dispatch_Id") or r.get("Correlation_Id"))
            print("| kernel | counter | dispatches | sum | per dispatch |")
            print("|---|---|---:|---:|---:|")
            for (name, cnt), (_, tot, ids) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
                print("| `%s` | %s | %d | %.6g | %.6g |" % (name, cnt, len(ids), tot, tot / max(1, len(ids))))
        else:
            print("| kernel | calls | total ns | average ns | % |")
            print("|---|---:|---:|---:|---:|")
            for r in rows:
                print("| `%s` | %s | %s | %s | %s |" % (r["Name"].split("(")[0], r["Calls"], r["TotalDurationNs"],
                                                   r["AverageNs"], r["Percentage"]))
        print()


def rocprof_gaps(path, top=12):
    """Print the level loop of the last enumeration in a rocprofv3 kernel_trace CSV
    (from the last k_root_init to the first ordering kernel): its span, the time at
    least one kernel runs, the time none does, and the longest gaps between kernels
    with the kernel and stream on each side."""
    import csv

    with open(path) as f:
        rows = list(csv.DictReader(f))
    ks = sorted(({"n": _short(r["Kernel_Name"]).replace("fcbo::", ""), "s": int(r["Start_Timestamp"]),
                  "e": int(r["End_Timestamp"]), "q": r.get("Stream_Id", "?")} for r in rows), key=lambda k: k["s"])
    roots = [i for i, k in enumerate(ks) if k["n"] == "k_root_init"]
    if not roots:
        raise SystemExit("no k_root_init dispatch in %s" % path)
    i0 = roots[-1]
    i1 = next((i for i in range(i0, len(ks)) if ks[i]["n"].startswith("k_subtree_size")), len(ks))
    loop = ks[i0:i1]
    t0, t1 = loop[0]["s"], (ks[i1]["s"] if i1 < len(ks) else max(k["e"] for k in loop))
    busy, gaps = 0, []
    cur_s, cur_e, last = loop[0]["s"], loop[0]["e"], loop[0]
    for k in loop[1:]:
        if k["s"] > cur_e:
            busy += cur_e - cur_s
            gaps.append((cur_e - t0, k["s"] - cur_e, last, k))
            cur_s, cur_e, last = k["s"], k["e"], k
        elif k["e"] > cur_e:
            cur_e, last = k["e"], k
    busy += cur_e - cur_s
    if t1 > cur_e:
        gaps.append((cur_e - t0, t1 - cur_e, last, ks[i1] if i1 < len(ks) else last))
    span = t1 - t0
    cross = [g for g in gaps if g[2]["q"] != g[3]["q"]]
    print("## Level loop of the last enumeration: time with no kernel running\n")
    print("| span us | some kernel running us | no kernel running us | gaps | gaps across streams | their us |")
    print("|---:|---:|---:|---:|---:|---:|")
    print("| %.1f | %.1f | %.1f | %d | %d | %.1f |\n" % (span / 1e3, busy / 1e3, (span - busy) / 1e3, len(gaps),
                                                         len(cross), sum(g[1] for g in cross) / 1e3))
    print("| at us | gap us | after (stream) | before (stream) |")
    print("|---:|---:|---|---|")
    for at, gap, a, b in sorted(gaps, key=lambda g: -g[1])[:top]:
        print("| %.1f | %.1f | `%s` (%s) | `%s` (%s) |" % (at / 1e3, gap / 1e3, a["n"], a["q"], b["n"], b["q"]))
    print()


def _counter_rows(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name):
    return name.split("(")[0].replace("void ", "")


def rocprof_traffic(fetch_csv, write_csv, enumerations, output_launches, copy_gib):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of one bench process, scaled by
    what they read for the plain copy (FETCH) and fill (WRITE) of `copy_gib` GiB run
    first, per kernel per dispatch; plus the records bench.py reads: the output
    kernels per launch, the level loop per enumeration."""
    nbytes = copy_gib * (1 << 30)
    per = {}
    factors = {}
    for which, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        calib = None
        for r in rows:
            name = r["Kernel_Name"]
            if which == "FETCH_SIZE" and "copy" in name.lower() and calib is None:
                calib = float(r["Counter_Value"]) * 1024
            if which == "WRITE_SIZE" and "FillFunctor" in name and calib is None:
                calib = float(r["Counter_Value"]) * 1024
        factors[which] = nbytes / calib
        for r in rows:
            name = _short(r["Kernel_Name"])
            if not name.startswith("fcbo::"):
                continue
            d = per.setdefault(name, {"FETCH_SIZE": [], "WRITE_SIZE": []})
            d[which].append(float(r["Counter_Value"]) * 1024 * factors[which])
    print("Calibration: the %g GiB copy reads %.3f x its bytes in FETCH_SIZE (factor %.3f); the %g GiB fill "
          "writes %.3f x in WRITE_SIZE (factor %.3f).\n" % (copy_gib, 1 / factors["FETCH_SIZE"], factors["FETCH_SIZE"],
                                                           copy_gib, 1 / factors["WRITE_SIZE"], factors["WRITE_SIZE"]))
    print("| kernel | dispatches | fetch GB per dispatch | write GB per dispatch | fetch GB per step | write GB per step |")
    print("|---|---:|---:|---:|---:|---:|")
    loop_f = loop_w = 0.0
    out_f = out_w = 0.0
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1]["FETCH_SIZE"]) - sum(kv[1]["WRITE_SIZE"])):
        n = max(len(d["FETCH_SIZE"]), 1)
        f, w = sum(d["FETCH_SIZE"]), sum(d["WRITE_SIZE"])
        base = name.split("::")[1].split("<")[0]
        if base in ("k_output_block", "k_output_intents"):
            out_f += f / output_launches
            out_w += w / output_launches
            steps = output_launches
        else:
            steps = enumerations
            if base in LEVEL_LOOP_KERNELS:
                loop_f += f / enumerations
                loop_w += w / enumerations
        print("| `%s` | %d | %.4f | %.4f | %.4f | %.4f |" % (name, n, f / n / 1e9, w / n / 1e9, f / steps / 1e9,
                                                          w / steps / 1e9))
    print()
    return out_f, out_w, loop_f, loop_w


def rocprof_sq(a_csv, b_csv, n_cu=256, ghz=2.4):
    """VALU issue share, wait share and LDS bank conflicts per kernel from the two SQ passes;
    returns the issue shares and the VALU wave-instruction counts by kernel."""
    agg = {}
    for path in (a_csv, b_csv):
        for r in _counter_rows(path):
            name = _short(r["Kernel_Name"])
            if not name.startswith("fcbo::"):
                continue
            d = agg.setdefault(name, {"ns": {}, "c": {}})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            key = (path, r["Dispatch_Id"])
            d["ns"][key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    print("| kernel | ms | VALU instr | VALU issue | LDS instr | VALU active | waiting | LDS bank conflict cycles |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    issue, valu_by = {}, {}
    for name, d in sorted(agg.items(), key=lambda kv: -sum(v for (p, _), v in kv[1]["ns"].items() if p == a_csv)):
        c = d["c"]
        ms = sum(v for (p, _), v in d["ns"].items() if p == a_csv) / 1e6
        valu = c.get("SQ_INSTS_VALU", 0.0)
        frac = valu * 4 / (ms * 1e-3 * ghz * 1e9 * n_cu * 4) if ms else 0.0
        cyc = c.get("SQ_WAVE_CYCLES", 0.0)
        active = c.get("SQ_ACTIVE_INST_VALU", 0.0) / cyc if cyc else 0.0
        wait = c.get("SQ_WAIT_ANY", 0.0) / cyc if cyc else 0.0
        issue[name.split("::")[1]] = round(frac, 3)
        valu_by[name.split("::")[1]] = valu
        print("| `%s` | %.3f | %.3g | %.2f | %.3g | %.2f | %.2f | %.3g |" % (
            name, ms, valu, frac, c.get("SQ_INSTS_LDS", 0.0), active, wait, c.get("SQ_LDS_BANK_CONFLICT", 0.0)))
    print()
    return issue, valu_by


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="ctx50000x400")
    ap.add_argument("--extents", choices=("auto", "yes", "no"), default="auto",
                    help="write the extent bitmaps (auto: when K x N/8 bytes fit in a third of device memory)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-cover", action="store_true", help="skip the cover-edge measurement")
    ap.add_argument("--host-stream-rows", type=int, default=1 << 20,
                    help="rows of the ordered output streamed to pinned host memory after the steps (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="threads of the all-core CPU baseline (0: the "
                    "process's cores, at most 16)")
    ap.add_argument("--cpu-bitmap-tests", type=int, default=2_000_000,
                    help="closure-test budget of the bitmap oracle's prefix (0: skip)")
    ap.add_argument("--pool-steps", type=int, default=3, help="timed steps of the task-pool schedule (0: skip)")
    ap.add_argument("--schedule", choices=("level", "pool"), default="level",
                    help="schedule of the timed steps: level sync, or the task pool (then no separate pool run)")
    ap.add_argument("--bounded-frac", type=float, default=0.25,
                    help="bounded run: memory limit as a fraction of the unbounded step's peak (0: skip)")
    ap.add_argument("--bounded-gib", type=float, default=0.0, help="bounded run: memory limit in GiB (overrides "
                    "--bounded-frac)")
    ap.add_argument("--bounded-extents", choices=("yes", "no"), default="yes")
    ap.add_argument("--bounded-piece-rows", type=int, default=1 << 20)
    ap.add_argument("--bounded-runs", type=int, default=2, help="bounded runs; the last one is reported")
    ap.add_argument("--hbm-probe-gib", type=float, default=4.0)
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="run one device-to-device copy of this size first (counter calibration)")
    ap.add_argument("--rocprof-summary", nargs="+", metavar="CSV")
    ap.add_argument("--rocprof-gaps", metavar="KERNEL_TRACE_CSV",
                    help="idle time between kernels in the last enumeration's level loop")
    ap.add_argument("--rocprof-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--rocprof-sq", nargs=2, metavar=("SQ_A_CSV", "SQ_B_CSV"))
    ap.add_argument("--enumerations", type=int, default=3, help="enumerations in the profiled process")
    ap.add_argument("--output-launches", type=int, default=2, help="output phases in the profiled process")
    ap.add_argument("--intents-only", action="store_true",
                    help="the profiled process wrote intents only (its output record is output_intents)")
    args = ap.parse_args()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return
    if args.rocprof_gaps:
        rocprof_gaps(args.rocprof_gaps)
        return
    if args.rocprof_traffic or args.rocprof_sq:
        sha = source_sha256()
        issue, valu_by = rocprof_sq(*args.rocprof_sq) if args.rocprof_sq else (None, None)
        if args.rocprof_traffic:
            of, ow, lf, lw = rocprof_traffic(*args.rocprof_traffic, args.enumerations, args.output_launches,
                                             args.copy_probe_gib or 1.0)
            print("```")
            if args.intents_only:
                print("traffic-record: class=output_intents kernel=k_output_intents source_sha256=%s "
                      "fetch_bytes_per_launch=%d write_bytes_per_launch=%d" % (sha, of, ow))
            else:
                print("traffic-record: class=output kernel=k_output_intents+k_output_block source_sha256=%s "
                      "fetch_bytes_per_launch=%d write_bytes_per_launch=%d" % (sha, of, ow))
            loop_issue = {k: v for k, v in (issue or {}).items() if k.split("<")[0] in LEVEL_LOOP_KERNELS}
            extra = " valu_issue=%s" % json.dumps(loop_issue, separators=(",", ":")) if loop_issue else ""
            if valu_by:
                loop_valu = sum(v for k, v in valu_by.items() if k.split("<")[0] in LEVEL_LOOP_KERNELS)
                extra += " valu_instr_per_step=%d" % int(loop_valu / args.enumerations)
            print("traffic-record: class=level_loop source_sha256=%s fetch_bytes_per_step=%d write_bytes_per_step=%d%s"
                  % (sha, lf, lw, extra))
            print("```")
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import synth

    n, m, _ = synth.CONFIGS[args.workload]
    if args.schedule == "pool" and m > 512:
        print("the task-pool schedule needs at most 512 attributes (%s has %d)" % (args.workload, m), file=sys.stderr)
        sys.exit(2)
    rows = synth.make_config(args.workload)
    wn, wm = (n + 63) // 64, (m + 63) // 64

    cpu = None
    if not args.no_cpu:
        threads = args.cpu_threads or min(16, len(host_cores()))
        cpu = cpu_baselines(rows, m, threads, args.cpu_bitmap_tests)
        print("[bench] cpu baseline: %s" % json.dumps(cpu), file=sys.stderr, flush=True)

    import torch

    import closed_set_enumeration_amd as fca

    if not torch.cuda.is_available():
        print("no HIP device", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    fca.load_library()
    if args.copy_probe_gib > 0:
        nel = int(args.copy_probe_gib * (1 << 30)) // 8
        src = torch.ones(nel, dtype=torch.int64, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy probe: %d bytes read, %d bytes written" % (nel * 8, nel * 8), file=sys.stderr, flush=True)
        del src, dst
    probe = hbm_probe(torch, args.hbm_probe_gib) if args.hbm_probe_gib > 0 else None

    ctx = fca.Context(rows, m)
    sched = fca.FCBO_TASK_POOL if args.schedule == "pool" else 0
    k = ctx.count(pool=bool(sched))
    if args.extents == "auto":
        free, _ = torch.cuda.mem_get_info()
        extents = k * wn * 8 <= free / 3
    else:
        extents = args.extents == "yes"
    ints, exts = ctx.alloc_outputs(k, extents)
    print("[bench] %s: K=%d, output buffers %.2f GB" % (args.workload, k, (ints.numel() + (exts.numel() if extents else 0)) * 8 / 1e9),
          file=sys.stderr, flush=True)
    if probe and extents:
        # the store rate this destination allows: a fill of the extent buffer itself
        # (a 30 GB buffer fills slower than the 4 GiB probe)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        best = None
        for _ in range(3):
            e[0].record()
            exts.zero_()
            e[1].record()
            torch.cuda.synchronize()
            best = e[0].elapsed_time(e[1]) if best is None else min(best, e[0].elapsed_time(e[1]))
        probe["output_buffer_fill"] = {"bytes": exts.numel() * 8, "ms": round(best, 4),
                                       "GBps": round(exts.numel() * 8 / (best * 1e-3) / 1e9, 1)}
    for i in range(args.warmup):
        rc, kk, st = ctx.enumerate_into(ints, exts, sched)
        assert rc == fca.FCBO_OK and kk == k
        print("[bench] warmup %d: %.3f ms" % (i, st["enumerate_ms"]), file=sys.stderr, flush=True)
    # per-kernel-class breakdown: one untimed step with an event pair around every kernel class
    rc, kk, prof = ctx.enumerate_into(ints, exts, sched | fca.FCBO_PROFILE)
    assert rc == fca.FCBO_OK and kk == k
    print("[bench] profiled step: %.3f ms" % prof["enumerate_ms"], file=sys.stderr, flush=True)

    per_step = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        rc, kk, st = ctx.enumerate_into(ints, exts, sched)
        assert rc == fca.FCBO_OK and kk == k
        per_step.append(st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    print("[bench] timed %d steps: %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr, flush=True)

    def avg(key):
        return sum(s[key] for s in per_step) / len(per_step)

    st0 = per_step[-1]
    kernel_ms = dict(prof["kernel_ms"])
    launches = dict(prof["kernel_launches"])
    records = profile_records(args.workload)

    # the dominant kernel class: the output writer, one launch per step, timed
    # live on every timed step (the output phase is its kernels alone)
    out_bytes = kernel_bytes("output", st0, wm, wn, n, k, extents)
    out_ms = avg("output_ms")
    achieved = out_bytes / (out_ms * 1e-3) / 1e9
    rec = records.get("output" if extents else "output_intents")
    roof = {"kernel": "output", "bound": "hbm",
            "kernels": ["k_output_intents", "k_output_block"] if extents else ["k_output_intents"],
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (int(rec["fetch_bytes_per_launch"]) + int(rec["write_bytes_per_launch"])) if rec else None,
            "bytes_per_launch": int(out_bytes), "avg_launch_ms": round(out_ms, 4),
            "frac_of_fill_probe": round(achieved / probe["fill_GBps"], 4) if probe else None,
            "frac_of_output_buffer_fill": (round(achieved / probe["output_buffer_fill"]["GBps"], 4)
                                           if probe and "output_buffer_fill" in probe else None),
            "timing": "timed steps, HIP events around the output phase"}

    # the closure kernels: the level loop against the model byte count
    loop_ms = avg("closure_kernel_ms")
    model = st0["model_bytes"]
    loop_gbs = model / (loop_ms * 1e-3) / 1e9
    lrec = records.get("level_loop")
    closure_roof = {
        "kernels": "level loop: root, closure tests, scans, child writes, per-level host wait",
        "bound": "hbm", "model_bytes": int(model), "ms": round(loop_ms, 4), "achieved": round(loop_gbs, 1),
        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(loop_gbs / HBM_PEAK_GBS, 4),
        "traffic": (int(lrec["fetch_bytes_per_step"]) + int(lrec["write_bytes_per_step"])) if lrec else None,
        "valu_issue": json.loads(lrec["valu_issue"]) if lrec and "valu_issue" in lrec else None,
        "timing": "timed steps, HIP events around the level loop"}
    if closure_roof["traffic"]:
        closure_roof["traffic_over_model"] = round(closure_roof["traffic"] / model, 3)
    # The level loop's kernels are bound by vector-instruction issue, not HBM: their
    # VALU wave-instructions per step (counter pass of the same sources) over the
    # measured level loop, against the chip's issue rate, 256 CUs x 4 SIMDs x 2.4 GHz
    # / 4 cycles per wave64 instruction = 614.4 G/s (some instructions issue faster,
    # so this is the common-case peak)
    if lrec and "valu_instr_per_step" in lrec:
        vps = int(lrec["valu_instr_per_step"]) / (loop_ms * 1e-3) / 1e9
        closure_roof["alu"] = {"bound": "alu", "achieved": round(vps, 1), "peak": VALU_ISSUE_PEAK_G,
                               "unit": "G VALU wave-instructions/s", "frac": round(vps / VALU_ISSUE_PEAK_G, 4),
                               "valu_instr_per_step": int(lrec["valu_instr_per_step"])}

    # the same step with the task-pool schedule (M <= 512), on a context of its
    # own so that the timed context keeps its result and its memory
    task_pool = None
    if args.pool_steps > 0 and m <= 512 and not sched:
        free_before_pool = int(torch.cuda.mem_get_info()[0])
        pctx = None
        try:
            pctx = fca.Context(rows, m)
            rc, kk, pprof = pctx.enumerate_into(ints, exts, fca.FCBO_TASK_POOL | fca.FCBO_PROFILE)
            assert rc == fca.FCBO_OK and kk == k
            rc, kk, _ = pctx.enumerate_into(ints, exts, fca.FCBO_TASK_POOL)
            pst = []
            torch.cuda.synchronize()
            tp0 = time.perf_counter()
            for i in range(args.pool_steps):
                rc, kk, sp = pctx.enumerate_into(ints, exts, fca.FCBO_TASK_POOL)
                assert rc == fca.FCBO_OK and kk == k and sp["closure_tests"] == st0["closure_tests"]
                pst.append(sp)
            torch.cuda.synchronize()
            pms = (time.perf_counter() - tp0) * 1e3 / args.pool_steps

            def pavg(key):
                return sum(x[key] for x in pst) / len(pst)

            task_pool = {"ms_per_step": round(pms, 4), "concepts_per_s": round(k / (pms * 1e-3), 1),
                         "closure_tests_per_s": round(st0["closure_tests"] / (pms * 1e-3), 1),
                         "level_sync_ms_per_step": round(ms_per_step, 4),
                         "speedup_over_level_sync": round(ms_per_step / pms, 3),
                         "device_ms": {"enumerate": round(pavg("enumerate_ms"), 4),
                                       "level_loop_and_pool": round(pavg("closure_kernel_ms"), 4),
                                       "sort": round(pavg("sort_ms"), 4), "output": round(pavg("output_ms"), 4)},
                         "kernel_ms": {c: round(v, 4) for c, v in pprof["kernel_ms"].items()},
                         "kernel_ms_note": "one untimed profiled step; the pool kernel is counted under test_local, "
                                           "its commit under write_local",
                         "peak_device_bytes": int(pst[-1]["peak_device_bytes"]),
                         "steps": args.pool_steps}
        except (fca.FcboError, torch.OutOfMemoryError) as err:
            free, total = torch.cuda.mem_get_info()
            task_pool = {"error": str(err).splitlines()[0][:160], "device_free_bytes": int(free),
                         "device_total_bytes": int(total)}
        finally:
            if pctx is not None:
                pctx.close()
        if task_pool and "error" in task_pool:
            task_pool["device_free_bytes_before"] = free_before_pool
            task_pool["device_free_bytes_after_close"] = int(torch.cuda.mem_get_info()[0])
            task_pool["torch_reserved_bytes"] = int(torch.cuda.memory_reserved())
        print("[bench] task pool: %s" % json.dumps(task_pool), file=sys.stderr, flush=True)

    # the ordered output streamed to pinned host memory through two staging
    # buffers (not part of the step; includes the PCIe transfer)
    stream_host = None
    if args.host_stream_rows > 0:
        nrow = min(args.host_stream_rows, k)
        hi = torch.empty((nrow, wm), dtype=torch.int64).pin_memory()
        he = torch.empty((nrow, wn), dtype=torch.int64).pin_memory() if extents else None
        try:
            ctx.copy_to_host(0, nrow, hi, he, staging_rows=1 << 18)
            t_h = ctx.copy_to_host(0, nrow, hi, he, staging_rows=1 << 18)
            nb = nrow * 8 * (wm + (wn if extents else 0))
            stream_host = {"rows": nrow, "bytes": nb, "ms": round(t_h, 3),
                           "GBps": round(nb / (t_h * 1e-3) / 1e9, 1), "staging_rows": 1 << 18,
                           "timing": "second call, HIP events; device-to-host over PCIe"}
        except fca.FcboError as err:
            stream_host = {"error": str(err).splitlines()[0][:160],
                           "device_free_bytes": int(torch.cuda.mem_get_info()[0])}
        del hi, he
        print("[bench] host stream: %s" % json.dumps(stream_host), file=sys.stderr, flush=True)

    # the lattice's cover edges of the same result (not part of the step)
    cover = None
    if not args.no_cover:
        del ints, exts
        ints = exts = None
        torch.cuda.empty_cache()
        try:
            # the first cover computation of the last timed step's result: the
            # counting call and the writing call (HIP events on the stream)
            _, e, cms = ctx.cover_edges()
            cover = {"edges": int(e.shape[0]), "ms": round(cms, 4),
                     "edges_per_s": round(e.shape[0] / (cms * 1e-3), 1),
                     "concepts_per_s": round(k / (cms * 1e-3), 1),
                     "timing": "counting + writing call on the last step's result, HIP events"}
            del e
        except (fca.FcboError, torch.OutOfMemoryError) as err:
            cover = {"error": str(err).splitlines()[0][:160]}
        print("[bench] cover edges: %s" % json.dumps(cover), file=sys.stderr, flush=True)

    # the same enumeration in bounded device memory, every output row handed
    # to a sink (not part of the step)
    bounded = None
    if args.bounded_gib > 0 or args.bounded_frac > 0:
        ints = exts = None
        torch.cuda.empty_cache()
        peak = int(st0["peak_device_bytes"])
        limit = int(args.bounded_gib * (1 << 30)) if args.bounded_gib > 0 else int(peak * args.bounded_frac)
        ext_b = args.bounded_extents == "yes"
        try:
            ctx.set_memory_limit(limit)
            for _ in range(max(1, args.bounded_runs)):
                kb, stb = ctx.enumerate_bounded(lambda first, i, e: None, piece_rows=args.bounded_piece_rows,
                                                intents=True, extents=ext_b)
                assert kb == k
            ms_b = stb["enumerate_ms"]
            bounded = {"limit_bytes": limit, "unbounded_peak_bytes": peak, "peak_bytes": int(stb["peak_device_bytes"]),
                       "extents_out": ext_b, "piece_rows": args.bounded_piece_rows,
                       "output_bytes": int(stb["output_bytes"]), "batches": int(stb["batches"]),
                       "retries": int(stb["batch_retries"]), "splits": int(stb["batch_splits"]),
                       "ms": round(ms_b, 3), "concepts_per_s": round(k / (ms_b * 1e-3), 1),
                       "closure_tests_per_s": round(stb["closure_tests"] / (ms_b * 1e-3), 1),
                       "device_ms": {"level_loop": round(stb["closure_kernel_ms"], 3),
                                     "order": round(stb["sort_ms"], 3), "output": round(stb["output_ms"], 3)},
                       "timing": "host wall time of the last of %d calls, no-op sink" % max(1, args.bounded_runs)}
        except (fca.FcboError, torch.OutOfMemoryError) as err:
            bounded = {"limit_bytes": limit, "error": str(err).splitlines()[0][:160]}
        ctx.set_memory_limit(0)
        print("[bench] bounded: %s" % json.dumps(bounded), file=sys.stderr, flush=True)

    tests = st0["closure_tests"]
    out = {
        "metric": "concepts/sec and closure tests/sec at 1 GPU; % of HBM roofline",
        "value": round(k / (ms_per_step * 1e-3), 1),
        "unit": "concepts/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u64",
        "data": "synthetic",
        "config": {"workload": args.workload, "objects": n, "attributes": m, "extents_out": extents,
                   "concepts": k, "closure_tests": tests, "levels": st0["n_levels"],
                   "schedule": "task_pool" if sched else "level_sync"},
        "closure_tests_per_s": round(tests / (ms_per_step * 1e-3), 1),
        "device_ms": {"enumerate": round(avg("enumerate_ms"), 4), "level_loop": round(loop_ms, 4),
                      "sort": round(avg("sort_ms"), 4), "output": round(out_ms, 4)},
        "kernel_ms": {c: round(v, 4) for c, v in kernel_ms.items()},
        "kernel_launches": launches,
        "kernel_ms_from": "one untimed step with per-kernel events (%.3f ms)" % prof["enumerate_ms"],
        "roofline": roof,
        "closure_roofline": closure_roof,
        "column_streaming_what_if": column_streaming_what_if(args.workload, loop_ms),
        "hbm_probe": probe,
        "cpu_baseline": cpu["one"] if cpu else None,
        "cpu_baseline_all_cores": cpu["all"] if cpu else None,
        "cpu_baseline_bitmap_oracle": cpu.get("bitmap") if cpu else None,
        "cover_edges": cover,
        "host_stream": stream_host,
        "task_pool": task_pool,
        "bounded": bounded,
    }
    ctx.close()
    del ints, exts  # noqa: F821
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
