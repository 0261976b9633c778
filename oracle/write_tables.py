"""Write oracle/lloyd_max_tables.txt from the Lloyd-Max generator.

Run once:  python -m oracle.write_tables
"""
from __future__ import annotations

from .lloyd_max import TABLE_BITS, fp32_table
from .tables import TABLE_FILE, format_tables


def build() -> str:
    return format_tables({b: fp32_table(b) for b in TABLE_BITS})


if __name__ == "__main__":
    with open(TABLE_FILE, "w") as f:
        f.write(build())
    print("wrote", TABLE_FILE)
