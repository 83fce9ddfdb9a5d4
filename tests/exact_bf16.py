"""Exact-arithmetic bf16 checker used to pin the oracle (tests only).

It reaches the rounded sum by a route that shares nothing with the oracle's:
values are exact rationals (``fractions.Fraction``), the sum is exact, and the
nearest bf16 is found by searching the ordered list of finite bf16 values for
the neighbours of the sum and taking the nearer one, the one with the even
significand (even bit pattern) on a tie -- IEEE 754 roundTiesToEven stated as
a search rather than as arithmetic on exponents.  Slow; tiny inputs only.
"""
from __future__ import annotations

from fractions import Fraction

INF = "inf"
NEG_INF = "-inf"


def value(h: int):
    """Exact value of a bf16 pattern: Fraction, or INF / NEG_INF."""
    sign = -1 if (h >> 15) & 1 else 1
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    if e == 0xFF:
        if f:
            raise ValueError("NaN pattern")
        return INF if sign > 0 else NEG_INF
    if e == 0:
        mag = Fraction(f, 2 ** 133)
    else:
        mag = Fraction(128 + f) * Fraction(2) ** (e - 127 - 7)
    return sign * mag


# Finite non-negative bf16 patterns 0x0000..0x7F7F are increasing in value.
_POS_VALUES = None


def _pos_values():
    global _POS_VALUES
    if _POS_VALUES is None:
        _POS_VALUES = [value(p) for p in range(0x7F80)]
    return _POS_VALUES


def round_exact(x) -> int:
    """Nearest bf16 pattern to an exact value (ties to the even pattern).

    Zero results keep the sign passed in as the special strings "+0"/"-0".
    """
    if x == INF:
        return 0x7F80
    if x == NEG_INF:
        return 0xFF80
    if x == "+0":
        return 0x0000
    if x == "-0":
        return 0x8000
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    vals = _pos_values()
    # largest p with vals[p] <= a
    lo, hi = 0, len(vals) - 1
    if a >= vals[hi]:
        p = hi
    else:
        while lo < hi:
            mid = (lo + hi + 1) // 2
            if vals[mid] <= a:
                lo = mid
            else:
                hi = mid - 1
        p = lo
    if vals[p] == a:
        return sign | p
    # upper neighbour; above the largest finite value it is 2^128 (infinity)
    up_val = vals[p + 1] if p + 1 < len(vals) else Fraction(2) ** 128
    d_lo = a - vals[p]
    d_hi = up_val - a
    if d_lo < d_hi or (d_lo == d_hi and p % 2 == 0):
        return sign | p
    q = p + 1
    return sign | (0x7F80 if q >= 0x7F80 else q)


def exact_sum(a: int, b: int) -> int:
    """bf16 pattern of the exact sum a + b, rounded once (ties to even)."""
    va, vb = value(a), value(b)
    if va in (INF, NEG_INF) or vb in (INF, NEG_INF):
        infs = {v for v in (va, vb) if v in (INF, NEG_INF)}
        if len(infs) == 2:
            raise ValueError("inf + -inf is NaN")
        return round_exact(infs.pop())
    s = va + vb
    if s == 0:
        # IEEE 754: an exact zero sum is +0 under roundTiesToEven unless both
        # operands are -0.
        both_neg_zero = (a == 0x8000) and (b == 0x8000)
        return round_exact("-0" if both_neg_zero else "+0")
    return round_exact(s)


def compare_key(h: int):
    """Total order key of a non-NaN bf16 for max-finding: -0 equals +0."""
    v = value(h)
    if v == INF:
        return (2, 0)
    if v == NEG_INF:
        return (0, 0)
    return (1, v)


def first_argmax(base_row, bias_row) -> int:
    """Lowest index of the maximum of the exact-rounded sums."""
    best_i, best_k = None, None
    for i, (a, b) in enumerate(zip(base_row, bias_row)):
        k = compare_key(exact_sum(int(a), int(b)))
        if best_k is None or k > best_k:
            best_i, best_k = i, k
    return best_i
