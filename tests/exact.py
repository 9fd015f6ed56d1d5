"""Exact-arithmetic helpers for pinning the oracle (Python integers and Fractions only)."""
from fractions import Fraction

import numpy as np


def f32_nearest(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) binary32 value of a rational, normal range."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]

    def key(v):
        v = np.float32(v)
        return (abs(Fraction(float(v)) - fr), int(v.view(np.uint32)) & 1)

    return np.float32(min(cands, key=key))


def frac(x) -> Fraction:
    return Fraction(float(x))


def ulp32(x: float) -> float:
    x = np.float32(abs(x))
    return float(np.nextafter(x, np.float32(np.inf)) - x)
