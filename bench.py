"""Benchmark: concept enumeration throughput on one MI355X.

One step = one full call of fcbo_enumerate on the seeded 50,000 x 400 context:
root, every level of closure tests and child writes, the output ordering and the
ordered intents plus extent bitmaps written to preallocated device buffers.
Inputs (the context) are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps 5] [--warmup 1] [--workload ctx50000x400]

Prints one JSON line.  `value` is concepts per second; closure tests per
second, per-kernel-class times (HIP events), the roofline of the dominant kernel
and the CPU oracle timed on a bounded sample are added.

The timed steps run without per-kernel events (recording an event pair around
every kernel class costs about 0.6 ms a step on the 50,000 x 400 context); the
library still times its phases with HIP events on its stream, and the output
phase is the output kernels alone (with extents: the intent gather, then the
row-block extent kernel), so the roofline's duration for them is measured live
on every timed step.  The per-class breakdown
(`kernel_ms`) comes from one extra, untimed step with per-kernel events.  Parts
of a level run on the library's side streams, so the times of the classes that
overlap there (mid and huge tests, the writers) include waiting and add up to
more than the level loop; the output kernel runs alone.
`closure_column_equivalent` restates the whole level loop's speed (all tests,
scans and child writes, wall time) in the terms of a column-streaming closure:
the bandwidth such a kernel would need to make the same closure tests in that
time.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s


def kernel_bytes(cls, st, wm, wn, n, k, extents):
    """Algorithmic bytes one step moves in a kernel class."""
    if cls == "test_local":
        # per parent: intent, cursor, two list offsets in; pass mask, child and object counts out;
        # per object of the extent: its list entry and its row
        return (st["local_parents"] * (8 * wm + 4 + 16 + 8 * wm + 8)
                + st["local_parent_objects"] * (4 + 8 * wm))
    if cls == "test_medium":
        return (st["medium_parents"] * (4 + 8 * wm + 4 + 16 + 8 * wm + 8)
                + st["medium_parent_objects"] * (4 + 8 * wm))
    if cls == "test_big":
        # per test: task, parent index, intent, list offsets, result; per list entry read: entry and column word
        return st["big_tests"] * (8 + 4 + 8 * wm + 16 + 4) + st["big_scanned_objects"] * (4 + 8)
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


def measured_traffic(cls, workload):
    """HBM bytes per launch of a kernel class from the committed rocprofv3 counter summary,
    or None when there is none or the device sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "%s_output_traffic.md" % workload)
    if not os.path.exists(path):
        return None
    sha = source_sha256()
    with open(path) as f:
        for line in f:
            if not line.startswith("traffic-record:"):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[1:])
            if kv.get("class") == cls and kv.get("source_sha256") == sha:
                return int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
    return None


def column_stream_equivalent(workload, closure_ms):
    """Bandwidth a column-streaming closure kernel would need for the same closure
    tests in `closure_ms` (the level loop's wall time): each test reads the non-zero
    words of the parent extent (8 bytes each; the oracle's sum_nzw, stored by
    tests/golden/make_golden.py) once."""
    path = os.path.join(ROOT, "tests", "golden", "%s.json" % workload)
    if not os.path.exists(path) or closure_ms <= 0:
        return None
    with open(path) as f:
        g = json.load(f)
    if "sum_nzw" not in g:
        return None
    gbytes = 8.0 * g["sum_nzw"] / 1e9
    gbs = gbytes / (closure_ms * 1e-3)
    return {"bytes_GB": round(gbytes, 2), "closure_ms": round(closure_ms, 4), "equivalent_GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "time": "level loop, wall"}


def cpu_baseline(rows, m, max_tests):
    import oracle

    t0 = time.perf_counter()
    r = oracle.cbo(rows, m, keep_extents=False, max_tests=max_tests)
    wall = time.perf_counter() - t0
    secs = r.seconds_enum + r.seconds_sort
    return {
        "value": r.n_concepts / secs,
        "unit": "concepts/s",
        "closure_tests_per_s": r.tests / secs,
        "cores": 1,
        "kind": "oracle",
        "sample": "serial CbO oracle, depth-first prefix of the same workload stopped after %d closure tests "
                  "(%d concepts, %.1f s enumerate+sort, %.1f s wall)" % (r.tests, r.n_concepts, secs, wall),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="ctx50000x400")
    ap.add_argument("--no-extents", action="store_true")
    ap.add_argument("--cpu-tests", type=int, default=8_000_000, help="closure-test budget of the CPU sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="run one device-to-device copy of this size first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import closed_set_enumeration_amd as fca
    import synth

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
    n, m, _ = synth.CONFIGS[args.workload]
    rows = synth.make_config(args.workload)
    extents = not args.no_extents
    wn, wm = (n + 63) // 64, (m + 63) // 64

    ctx = fca.Context(rows, m)
    k = ctx.count()
    ints, exts = ctx.alloc_outputs(k, extents)
    print("[bench] %s: K=%d, output buffers %.2f GB" % (args.workload, k, (ints.numel() + (exts.numel() if extents else 0)) * 8 / 1e9),
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        rc, kk, st = ctx.enumerate_into(ints, exts, 0)
        assert rc == fca.FCBO_OK and kk == k
        print("[bench] warmup %d: %.3f ms" % (i, st["enumerate_ms"]), file=sys.stderr, flush=True)
    # per-kernel-class breakdown: one untimed step with an event pair around every kernel class
    rc, kk, prof = ctx.enumerate_into(ints, exts, fca.FCBO_PROFILE)
    assert rc == fca.FCBO_OK and kk == k
    print("[bench] profiled step: %.3f ms" % prof["enumerate_ms"], file=sys.stderr, flush=True)

    per_step = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        rc, kk, st = ctx.enumerate_into(ints, exts, 0)
        assert rc == fca.FCBO_OK and kk == k
        per_step.append(st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    print("[bench] timed %d steps: %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr, flush=True)

    st0 = per_step[-1]
    kernel_ms = dict(prof["kernel_ms"])
    launches = dict(prof["kernel_launches"])
    dominant = max(kernel_ms, key=kernel_ms.get)
    roof = None
    b = kernel_bytes(dominant, st0, wm, wn, n, k, extents)
    if b is not None and launches[dominant] > 0:
        per_launch_bytes = b / launches[dominant]
        if dominant == "output" and launches[dominant] == 1:
            # the output phase of every timed step is the output kernels alone (HIP events on its stream)
            avg_ms = sum(s["output_ms"] for s in per_step) / args.steps
        else:
            avg_ms = kernel_ms[dominant] / launches[dominant]
        achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm",
                "kernels": (["k_output_intents", "k_output_block"] if extents else ["k_output_intents"])
                if dominant == "output" else None, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dominant, args.workload),
                "bytes_per_launch": int(per_launch_bytes), "avg_launch_ms": round(avg_ms, 4),
                "timing": "timed steps, HIP events around the output phase" if dominant == "output"
                          else "profiled step, HIP events per kernel class"}

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
                   "concepts": k, "closure_tests": tests, "levels": st0["n_levels"]},
        "closure_tests_per_s": round(tests / (ms_per_step * 1e-3), 1),
        "device_ms": {"enumerate": round(sum(s["enumerate_ms"] for s in per_step) / args.steps, 4),
                      "levels": round(sum(s["levels_ms"] for s in per_step) / args.steps, 4),
                      "order": round(sum(s["order_ms"] for s in per_step) / args.steps, 4),
                      "output": round(sum(s["output_ms"] for s in per_step) / args.steps, 4)},
        "kernel_ms": {c: round(v, 4) for c, v in kernel_ms.items()},
        "kernel_launches": launches,
        "kernel_ms_from": "one untimed step with per-kernel events (%.3f ms)" % prof["enumerate_ms"],
        "roofline": roof,
        "closure_column_equivalent": column_stream_equivalent(
            args.workload, sum(s["levels_ms"] for s in per_step) / args.steps),
        "cpu_baseline": None,
    }
    ctx.close()
    del ints, exts
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(rows, m, args.cpu_tests)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
