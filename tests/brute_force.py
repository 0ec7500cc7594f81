"""Exact brute-force GEMM for tiny inputs, independent of the oracle.

The sum is formed exactly with ``fractions.Fraction`` from values decoded by
numpy (not by the oracle's decoder), and rounded by searching the sorted
table of every finite binary16 value for the nearest one, ties to the
pattern with an even fraction field.  No floating-point arithmetic is
involved anywhere, so it pins the oracle's sum, its order-independence and
its rounding.
"""
from bisect import bisect_left
from fractions import Fraction
from functools import lru_cache

import numpy as np


@lru_cache(maxsize=1)
def _table():
    bits = np.arange(0x7C00, dtype=np.uint16)            # +0 .. largest finite
    vals = [Fraction(float(v)) for v in bits.view(np.float16).astype(np.float64)]
    return vals, [int(b) for b in bits]


def value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16).astype(np.float64)[0]))


def round_to_f16(x: Fraction) -> int:
    """Nearest binary16 bit pattern to the exact rational x, ties to even."""
    vals, bits = _table()
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    if a == 0:
        return sign
    top = vals[-1]
    # the binade above the largest finite value has spacing 2^5; at or above
    # top + 2^4 the nearest value would be 2^16, which is not finite -> inf
    if a >= top + Fraction(16):
        return sign | 0x7C00
    i = bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | bits[i]
    lo, hi = i - 1, min(i, len(vals) - 1)
    if a > top:
        return sign | bits[-1]
    dlo, dhi = a - vals[lo], vals[hi] - a
    if dlo < dhi:
        return sign | bits[lo]
    if dhi < dlo:
        return sign | bits[hi]
    return sign | (bits[lo] if bits[lo] % 2 == 0 else bits[hi])


def gemm(A_bits: np.ndarray, B_bits: np.ndarray, relu: bool = False, scale: Fraction = Fraction(1)) -> np.ndarray:
    """rne16(epi(scale * exact sum)); a zero result is returned as +0."""
    M, K = A_bits.shape
    K2, N = B_bits.shape
    assert K == K2
    a = [[value(int(A_bits[i, k])) for k in range(K)] for i in range(M)]
    b = [[value(int(B_bits[k, j])) for j in range(N)] for k in range(K)]
    out = np.zeros((M, N), dtype=np.uint16)
    for i in range(M):
        for j in range(N):
            s = scale * sum((a[i][k] * b[k][j] for k in range(K)), Fraction(0))
            if relu and s < 0:
                s = Fraction(0)
            out[i, j] = round_to_f16(s)
    return out
