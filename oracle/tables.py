"""Frozen Lloyd-Max codebooks used by the oracle (test infrastructure).

``lloyd_max_tables.txt`` holds, for each width, the float32 centroids and
boundaries as 32-bit hex patterns.  It is written by ``write_tables.py``,
which calls only ``lloyd_max.fp32_table``; a CPU test regenerates it and
checks it is unchanged.
"""
from __future__ import annotations

import functools
import os

import numpy as np

TABLE_FILE = os.path.join(os.path.dirname(__file__), "lloyd_max_tables.txt")


@functools.lru_cache(maxsize=None)
def _load():
    out = {}
    with open(TABLE_FILE) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *words = line.split()
            vals = np.array([int(w, 16) for w in words], dtype=np.uint32).view(np.float32)
            out[tag] = vals
    return out


def codebook(bits: int):
    """(centroids, boundaries) float32 arrays for a value width."""
    t = _load()
    return t[f"c{bits}"].copy(), t[f"b{bits}"].copy()


def format_tables(tables: dict) -> str:
    lines = ["# Lloyd-Max codebooks for N(0,1), float32 bit patterns.",
             "# cN: 2^N centroids ascending; bN: 2^N-1 boundaries ascending.",
             "# Written by oracle/write_tables.py (3-bit = the printed table)."]
    for bits in sorted(tables):
        cent, bnd = tables[bits]
        for tag, arr in (("c", cent), ("b", bnd)):
            words = " ".join(f"{int(w):08x}" for w in np.asarray(arr, np.float32).view(np.uint32))
            lines.append(f"{tag}{bits} {words}")
    return "\n".join(lines) + "\n"
