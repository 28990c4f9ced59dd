"""Reader for the hand-derived fixtures in tests/golden/*.txt."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(s):
    return [c == "1" for c in s]


def read_fixture(name):
    rows, concepts, info = [], [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "row":
                _, bits = rest.split()
                rows.append(_bits(bits))
            elif key == "concept":
                a, b = rest.split("|")
                concepts.append((_bits(a.strip()), _bits(b.strip())))
            elif key in ("level_concepts", "level_tests"):
                info[key] = [int(x) for x in rest.split()]
            else:
                info[key] = int(rest)
    cells = np.array(rows, dtype=bool)
    assert cells.shape == (info["objects"], info["attributes"])
    return cells, concepts, info
