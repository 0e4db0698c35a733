"""Pure-Python OCP E4M3FN codec (TEST INFRASTRUCTURE ONLY).

A second, independent statement of the format that pins the C oracle's codec.
Format (the FP8 E4M3 representation listed in tutorial 6 of the page
"vLLM：从 KV Cache 到高吞吐推理服务"; OCP 8-bit floating point spec, E4M3 flavour):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the
subnormals m * 2^-9; no infinities; S.1111.111 is NaN; the largest finite
magnitude is 1.75 * 2^8 = 448.

Encoding rounds to nearest with ties to the even code (the table of all finite
values is enumerated and the nearest is chosen, ties to the even code index),
saturating magnitudes above 448 (and infinity) to 448; NaN keeps its sign.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Optional

_TABLE: Optional[List[Fraction]] = None


def decode_exact(code: int) -> Optional[Fraction]:
    """Exact rational value of a code, None for NaN."""
    code &= 0xFF
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return None
    if e == 0:
        v = Fraction(m, 2 ** 9)
    else:
        v = Fraction(8 + m, 8) * (Fraction(2) ** (e - 7))
    return -v if s else v


def decode(code: int) -> float:
    v = decode_exact(code)
    if v is None:
        return math.nan
    return math.copysign(float(abs(v)), -1.0 if code & 0x80 else 1.0)


def _positive_table() -> List[Fraction]:
    global _TABLE
    if _TABLE is None:
        _TABLE = [decode_exact(c) for c in range(0x7F)]  # codes 0..126, ascending values
    return _TABLE


def encode(x: float) -> int:
    """Nearest code to x (ties to even code), saturating; by search over the value table."""
    if math.isnan(x):
        return 0xFF if math.copysign(1.0, x) < 0 else 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    if math.isinf(x):
        return sign | 0x7E
    a = Fraction(abs(x))
    tab = _positive_table()
    if a >= tab[-1]:
        return sign | 0x7E
    # find neighbours tab[i] <= a < tab[i+1]
    lo, hi = 0, len(tab) - 1
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if tab[mid] <= a:
            lo = mid
        else:
            hi = mid
    dlo, dhi = a - tab[lo], tab[hi] - a
    if dlo < dhi:
        c = lo
    elif dhi < dlo:
        c = hi
    else:
        c = lo if lo % 2 == 0 else hi   # even code = even mantissa
    return sign | c
