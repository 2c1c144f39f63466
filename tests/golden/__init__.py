"""Tiny parser for the golden fixtures (``key = value`` lines, ``#`` comments)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = val
    return out


def floats(s: str):
    return [float(t) for t in s.split()]


def ints(s: str):
    return [int(t) for t in s.split()]
