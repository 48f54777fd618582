"""Reader for the hand-worked text fixtures under tests/golden/."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def exact_f32(tokens) -> np.ndarray:
    """Parse exact rationals ("p/q", "-0") into binary32, asserting exactness."""
    out = np.zeros(len(tokens), np.float32)
    for i, t in enumerate(tokens):
        fr = Fraction(t)
        v = np.float32(float(fr))
        assert Fraction(float(v)) == fr, f"fixture value {t} is not binary32-exact"
        if t.startswith("-") and fr == 0:
            v = np.float32(-0.0)
        out[i] = v
    return out


def read_blocks(name: str) -> list[dict]:
    cases, cur = [], None
    with open(os.path.join(GOLDEN, name)) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
            elif key == "end":
                cases.append(cur)
                cur = None
            elif key in ("w", "deq"):
                cur[key] = exact_f32(vals)
            elif key == "scale":
                cur[key] = int(vals[0], 16)
            elif key == "codes":
                cur[key] = np.array([int(v) for v in vals], np.int64)
            elif key == "bytes":
                cur[key] = bytes(int(v, 16) for v in vals)
            else:
                raise ValueError(f"unknown fixture key {key}")
    return cases


def read_conversion_points() -> list[tuple[str, int, int]]:
    pts = []
    with open(os.path.join(GOLDEN, "conversion_points.txt")) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].split()
            if line:
                pts.append((line[0], int(line[1], 16), int(line[2], 16)))
    return pts
