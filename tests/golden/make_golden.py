"""Write the oracle's expected values for the full-size seeded workloads.

Runs only the CPU oracle (oracle/) on the named workloads and stores, per
workload, the concept count, closure tests, item pairs, per-level counts, the
byte-model sums and a SHA-256 of the sorted intent array.  The GPU tests
compare against these files; nothing here touches the GPU library.

    python tests/golden/make_golden.py ctx50000x400
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


def golden(name: str) -> dict:
    rows = synth.make_config(name)
    n, m, _ = synth.CONFIGS[name]
    t0 = time.time()
    r = oracle.cbo(rows, m, keep_extents=False)
    wall = time.time() - t0
    return {
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
        "intents_sha256": hashlib.sha256(np.ascontiguousarray(r.intents, dtype="<u8").tobytes()).hexdigest(),
        "oracle_enum_seconds": r.seconds_enum,
        "oracle_sort_seconds": r.seconds_sort,
        "oracle_wall_seconds": wall,
    }


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
