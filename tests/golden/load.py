"""Reader for the small text fixtures in this folder (values printed on the pages)."""
from __future__ import annotations

import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (x.strip() for x in line.split("=", 1))
            rows = [[float(t) for t in r.split()] for r in val.split("|")]
            out[key] = np.array(rows if len(rows) > 1 else rows[0], dtype=np.float64)
    return out
