"""Parsers for the hand-derived text fixtures in this folder."""
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def _num(tok: str) -> float:
    if "*" in tok:
        a, b = tok.split("*")
        return float(a) * float(b)
    return float(Fraction(tok))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (x.strip() for x in line.split("=", 1))
            out[key] = [_num(t) for t in val.split()]
    return out
