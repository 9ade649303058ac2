"""Exact rounding of rational numbers to binary16 / binary32, written with
Python Fractions and numpy's nextafter.  An independent second route to the
directed roundings the oracle performs with binary64 tricks."""
from __future__ import annotations

from fractions import Fraction as F

import numpy as np


def _down(x: F, t):
    f = t(float(x))
    while not np.isfinite(f) or F(float(f)) > x:
        f = np.nextafter(f, t(-np.inf))
    while True:
        n = np.nextafter(f, t(np.inf))
        if np.isfinite(n) and F(float(n)) <= x:
            f = n
        else:
            return f


def _up(x: F, t):
    f = t(float(x))
    while not np.isfinite(f) or F(float(f)) < x:
        f = np.nextafter(f, t(np.inf))
        if not np.isfinite(f):
            return f
    while True:
        p = np.nextafter(f, t(-np.inf))
        if F(float(p)) >= x:
            f = p
        else:
            return f


def rd32(x: F) -> np.float32:
    return _down(x, np.float32)


def ru32(x: F) -> np.float32:
    return _up(x, np.float32)


def rd16(x: F) -> np.float16:
    return _down(x, np.float16)


def ru16(x: F) -> np.float16:
    return _up(x, np.float16)


def rn32(x: F) -> np.float32:
    lo = rd32(x)
    if F(float(lo)) == x:
        return lo
    hi = np.nextafter(lo, np.float32(np.inf))
    dl, dh = x - F(float(lo)), F(float(hi)) - x
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (lo.view(np.uint32) & 1) == 0 else hi


def fr(x) -> F:
    return F(float(x))
