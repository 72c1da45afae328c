"""Reader for the hand-worked fixtures under tests/golden/.

Format: '#' lines are comments; a header line "<name> <rows> <cols>" is
followed by <rows> lines of <cols> whitespace-separated numbers (decimal, or
hexadecimal with a 0x prefix).
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    i = 0
    while i < len(lines):
        key, r, c = lines[i].split()
        r, c = int(r), int(c)
        rows = [[int(v, 16) if v.startswith("0x") else float(v)
                 for v in lines[i + 1 + q].split()] for q in range(r)]
        assert all(len(row) == c for row in rows), (name, key)
        out[key] = np.array(rows, dtype=object)
        i += 1 + r
    return out
