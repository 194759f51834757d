"""Reader for the small key/value text fixtures in this folder."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    """Return {key: list of rows}; each row is a list of numbers (int where possible)."""
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            row = [float(x) if ("." in x or "e" in x) else int(x) for x in vals]
            out.setdefault(key, []).append(row)
    return out


def arr(d, key, dtype=np.int64):
    rows = d[key]
    return np.asarray(rows[0] if len(rows) == 1 else rows, dtype=dtype)
