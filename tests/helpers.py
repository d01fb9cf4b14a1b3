"""Shared helpers for the test suite (fixture parsing, small structures)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    """Parse a golden fixture: ``key values...`` lines, ``mask`` / ``tiles BM BN`` grids."""
    out = {"tiles": {}}
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    i = 0
    while i < len(lines):
        parts = lines[i].split()
        key = parts[0]
        if key == "end":
            break
        if key in ("mask", "tiles"):
            grid = []
            i += 1
            while i < len(lines) and lines[i][0] in "012":
                grid.append([int(c) for c in lines[i]])
                i += 1
            if key == "mask":
                out["mask"] = grid
            else:
                out["tiles"][(int(parts[1]), int(parts[2]))] = grid
            continue
        out[key] = [int(x) for x in parts[1:]]
        i += 1
    return out
