"""Write the oracle's expected values for the full-size seeded workloads.

Runs only the CPU oracle (oracle/) on the named workloads and stores, per
workload, the concept count, closure tests, item pairs, per-level counts and
the byte-model sums, plus

* for workloads whose concepts fit in host memory: a SHA-256 of the sorted
  intent array and a SHA-256 of the array of extent hashes in the same order
  (oracle.cbo; the extent bitmaps themselves would not fit), and the class
  sums of the byte model;
* for every workload: the positional digests of the store-free search
  (oracle.cbo_digest, all host cores): intents and extents hashed and
  weighted by their output position, in total and per subtree of the root's
  children (consecutive ranges of the output);
* for the larger ones also the order-independent intent digest and slices:
  for a few attribute sets S, the sorted intents of the sub-context of the
  objects having all of S, which are exactly the workload's intents
  containing S (count and SHA-256).

The GPU tests compare against these files; nothing here touches the GPU
library.

    python tests/golden/make_golden.py ctx10000x128 ctx50000x400 ctx20000x256
"""

import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


# workloads checked through the store-free oracle, with their attribute slices
DIGEST_SLICES = {
    "ctx20000x256": [[149, 61], [139, 95], [3, 77], [10, 200, 255], [149]],
}


def sha_of(intents) -> str:
    return hashlib.sha256(np.ascontiguousarray(intents, dtype="<u8").tobytes()).hexdigest()


def positional(rows, m) -> dict:
    t0 = time.time()
    d = oracle.cbo_digest(rows, m, threads=os.cpu_count() or 1)
    wall = time.time() - t0
    return d, {
        "intent_digest": str(d.digest),
        "intent_positional": str(d.intent_positional),
        "extent_digest": str(d.extent_digest),
        "extent_positional": str(d.extent_positional),
        "root_children": [[c["attr"], c["size"], str(c["hi0"]), str(c["hi1"]), str(c["he0"]), str(c["he1"])]
                          for c in d.root_children],
        "digest_oracle_threads": d.threads,
        "digest_oracle_seconds": d.seconds,
        "digest_oracle_wall_seconds": wall,
    }


def golden_digest(name: str) -> dict:
    cells = synth.make_config(name, packed=False)
    rows = synth.pack_rows(cells)
    n, m, _ = synth.CONFIGS[name]
    d, pos = positional(rows, m)
    slices = []
    for attrs in DIGEST_SLICES[name]:
        sub = cells[cells[:, attrs].all(axis=1)]
        r = oracle.cbo(synth.pack_rows(sub), m, keep_extents=False)
        slices.append({"attributes": attrs, "objects": int(sub.shape[0]), "n_concepts": int(r.n_concepts),
                       "intents_sha256": sha_of(r.intents)})
    out = {
        "workload": name,
        "objects": n,
        "attributes": m,
        "generator_version": synth.GENERATOR_VERSION,
        "rows_sha256": synth.rows_sha256(rows),
        "n_concepts": int(d.n_concepts),
        "closure_tests": int(d.tests),
        "item_pairs": int(d.pairs),
        "sum_c": int(d.sum_c),
        "level_concepts": [int(x) for x in d.level_concepts],
        "level_tests": [int(x) for x in d.level_tests],
        "slices": slices,
        "oracle_wall_seconds": pos["digest_oracle_wall_seconds"],
    }
    out.update(pos)
    return out


def golden(name: str) -> dict:
    if name in DIGEST_SLICES:
        return golden_digest(name)
    rows = synth.make_config(name)
    n, m, _ = synth.CONFIGS[name]
    t0 = time.time()
    r = oracle.cbo(rows, m, keep_extents=False, hash_extents=True)
    wall = time.time() - t0
    d, pos = positional(rows, m)
    assert d.n_concepts == r.n_concepts and d.tests == r.tests
    out = {
        "workload": name,
        "objects": n,
        "attributes": m,
        "generator_version": synth.GENERATOR_VERSION,
        "rows_sha256": synth.rows_sha256(rows),
        "n_concepts": int(r.n_concepts),
        "closure_tests": int(r.tests),
        "item_pairs": int(r.pairs),
        "sum_nzw": int(r.sum_nzw),
        "sum_c": int(r.sum_c),
        "level_concepts": [int(x) for x in r.level_concepts],
        "level_tests": [int(x) for x in r.level_tests],
        "intents_sha256": sha_of(r.intents),
        "extent_hashes_sha256": sha_of(r.extent_hashes),
        "rowlocal_max": r.rowlocal_max,
        "sum_rl_objs": int(r.sum_rl_objs),
        "col_parents": int(r.col_parents),
        "col_nzw": int(r.col_nzw),
        "col_child_objs": int(r.col_child_objs),
        "model_bytes": int(oracle.model_bytes(r)),
        "oracle_enum_seconds": r.seconds_enum,
        "oracle_sort_seconds": r.seconds_sort,
        "oracle_wall_seconds": wall,
    }
    out.update(pos)
    return out


def main(names):
    for name in names:
        g = golden(name)
        path = os.path.join(HERE, name + ".json")
        with open(path, "w") as f:
            json.dump(g, f, indent=1)
            f.write("\n")
        print(path, g["n_concepts"], g["closure_tests"], "%.1fs" % g["oracle_wall_seconds"], flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["ctx50000x400"])
