"""Readers for the small text fixtures under tests/golden (each file cites its page)."""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_kv(name: str) -> dict[str, str]:
    """key = value lines; '#' starts a comment line; 'step ...' lines are kept in order."""
    out: dict[str, str] = {}
    steps = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("step "):
                steps.append(line.split()[1:])
                continue
            if "=" in line:
                k, v = line.split("=", 1)
                out[k.strip()] = v.strip()
            else:
                key, rest = line.split(None, 1)
                out[key] = rest
    if steps:
        out["_steps"] = steps  # type: ignore[assignment]
    return out


def matrix(text: str) -> np.ndarray:
    """'a b ; c d' -> 2x2 float array."""
    return np.array([[float(x) for x in row.split()] for row in text.split(";")], dtype=np.float64)


def vector(text: str) -> np.ndarray:
    return np.array([float(x) for x in text.split()], dtype=np.float64)


def exp_terms(text: str) -> float:
    """'c1,e1 c2,e2 ...' -> sum c * exp(e), evaluated in fp64."""
    total = 0.0
    for tok in text.split():
        c, e = tok.split(",")
        total += float(c) * math.exp(float(e))
    return total


def read_matrix_file(name: str) -> np.ndarray:
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([float(x) for x in line.split()])
    return np.array(rows, dtype=np.float64)
