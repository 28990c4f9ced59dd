"""Seeded synthetic formal contexts.

This package only draws and packs 0/1 object x attribute matrices.  It holds
none of the concept-enumeration arithmetic, so both the CPU oracle and the GPU
library can take their inputs from it without sharing any of the method.
"""

from .contexts import (  # noqa: F401
    CONFIGS,
    GENERATOR_VERSION,
    make_config,
    pack_rows,
    unpack_rows,
    random_context,
    words,
    rows_sha256,
    all_zero,
    all_ones,
    diagonal,
    contranominal,
    planted_bicluster,
    pad_with_full,
)
