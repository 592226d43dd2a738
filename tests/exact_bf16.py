"""Exact-arithmetic bf16 helpers for the tests (no floating point involved).

bf16 values are decoded from their bit fields into ``fractions.Fraction`` and
rounding is checked by its defining property -- the stored value is a
representable value nearest to the exact one, ties going to the even
significand -- by comparing against both neighbours.  Nothing here computes
a rounding the way the oracle or the kernels do, so these helpers can judge
both.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_INF_KEY = 0x7F80


def bf16_fraction(h: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    h = int(h) & 0xFFFF
    sign = -1 if h & 0x8000 else 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    if e == 0xFF:
        raise ValueError("non-finite bf16 0x%04x" % h)
    if e == 0:
        mag = Fraction(m, 1 << 7) / (Fraction(2) ** 126)
    else:
        mag = (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))
    return sign * mag


def _key(h: int) -> int:
    h = int(h) & 0xFFFF
    return -(h & 0x7FFF) if h & 0x8000 else h


def _unkey(k: int) -> int:
    return (0x8000 | (-k)) if k < 0 else k


def nearest_check(h: int, x: Fraction) -> str | None:
    """None if bf16 ``h`` is the round-to-nearest-even value of exact ``x``.

    Otherwise a short reason.  Only finite results are judged.
    """
    k = _key(h)
    if abs(k) >= _INF_KEY:
        return "non-finite result 0x%04x for %s" % (h, float(x))
    v = bf16_fraction(h)
    d = abs(x - v)
    for nk in (k - 1, k + 1):
        if abs(nk) >= _INF_KEY:
            continue
        dn = abs(x - bf16_fraction(_unkey(nk)))
        if dn < d:
            return "0x%04x (%r) is not nearest to %r" % (h, float(v), float(x))
        if dn == d and d != 0 and (int(h) & 1):
            return "tie at %r not resolved to even (got 0x%04x)" % (float(x), h)
    return None


def ulp_distance(a: int, b: int) -> int:
    """Number of bf16 steps between two finite bit patterns."""
    return abs(_key(a) - _key(b))


def bits_of(values) -> np.ndarray:
    """Exactly-representable float values -> bf16 bits (asserts exactness)."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (u >> 16).astype(np.uint16)
