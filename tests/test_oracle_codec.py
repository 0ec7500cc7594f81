"""Pins for the oracle's binary16 codec, against facts outside the oracle.

* numpy's float16 <-> float64 conversions (an independent, correctly rounded
  implementation) on every bit pattern and on 10^6 random doubles;
* IEEE 754 binary16 facts: round trip of every finite value, ties to even at
  every midpoint, the overflow threshold 65520 and the underflow tie 2^-25.
The tiled method writes fp16 "in the last copy" after an fp32 accumulator
("5分钟上手TileLang：GPU内核开发指南", section "避坑与调参"); these pins
fix the rounding that copy must perform.
"""
import math

import numpy as np
import pytest

import oracle

ALL = np.arange(65536, dtype=np.uint16)


def test_decode_matches_numpy_on_every_pattern():
    got = oracle.decode(ALL)
    ref = ALL.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros are kept
    assert math.copysign(1.0, got[0x8000]) == -1.0 and math.copysign(1.0, got[0]) == 1.0


def test_decode_known_values():
    # bit-field facts of binary16
    assert oracle.decode(np.array([0x3C00], np.uint16))[0] == 1.0
    assert oracle.decode(np.array([0x0001], np.uint16))[0] == 2.0 ** -24     # smallest subnormal
    assert oracle.decode(np.array([0x0400], np.uint16))[0] == 2.0 ** -14     # smallest normal
    assert oracle.decode(np.array([0x7BFF], np.uint16))[0] == 65504.0        # largest finite
    assert oracle.decode(np.array([0xC000], np.uint16))[0] == -2.0
    assert np.isinf(oracle.decode(np.array([0x7C00], np.uint16))[0])


def test_round_trip_every_finite_pattern():
    finite = ALL[np.isfinite(ALL.view(np.float16))]
    assert finite.size == 63488
    assert np.array_equal(oracle.encode(oracle.decode(finite)), finite)


def test_midpoints_round_to_even():
    pos = np.arange(0x0000, 0x7BFF, dtype=np.uint16)     # each with a finite successor
    lo = pos.view(np.float16).astype(np.float64)
    hi = (pos + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0                                 # exact in binary64
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    assert np.array_equal(oracle.encode(mid), even)
    assert np.array_equal(oracle.encode(-mid), even | 0x8000)
    # just off the midpoint the nearer neighbour wins
    assert np.array_equal(oracle.encode(np.nextafter(mid, np.inf)), (pos + 1).astype(np.uint16))
    assert np.array_equal(oracle.encode(np.nextafter(mid, -np.inf)), pos)


@pytest.mark.parametrize("x,bits", [
    (65519.99, 0x7BFF),            # below the overflow tie: largest finite
    (65520.0, 0x7C00),             # the tie between 65504 and 2^16 goes to infinity
    (-65520.0, 0xFC00),
    (1e300, 0x7C00),
    (2.0 ** -25, 0x0000),          # tie between 0 and 2^-24 goes to the even 0
    (-(2.0 ** -25), 0x8000),
    (2.0 ** -25 * 1.0001, 0x0001),
    (3 * 2.0 ** -25, 0x0002),      # tie between 2^-24 and 2^-23 goes to the even 2^-23
    (2.0 ** -14 - 2.0 ** -26, 0x0400),   # rounds up out of the subnormal range
    (2047.5 * 2.0 ** -10, 0x4000), # carry into the next binade: 1.99951171875 -> 2
    (0.0, 0x0000),
    (-0.0, 0x8000),
])
def test_encode_boundaries(x, bits):
    assert int(oracle.encode(np.array([x]))[0]) == bits


def test_encode_nan():
    out = oracle.encode(np.array([np.nan]))[0]
    assert np.isnan(np.array([out], np.uint16).view(np.float16)[0])


def test_encode_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(1234)
    n = 1_000_000
    x = rng.standard_normal(n) * np.exp2(rng.uniform(-30.0, 17.0, n))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode(x), ref)


def test_tolerance_rule():
    # ulp(r): 2^(max(E,1)-25) -- 2^-24 at zero/subnormals, 2^-10 in [1,2), 2^5 at the top binade
    r = np.array([0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x3BFF, 0x7BFF], np.uint16)
    u = oracle.ulp(r)
    assert list(u) == [2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -10, 2.0 ** -11, 2.0 ** 5]
    # |r| < 1: the 1e-3 absolute floor dominates
    ref = oracle.encode(np.array([0.25]))
    ok = oracle.encode(np.array([0.25 + 0.0009]))
    bad = oracle.encode(np.array([0.25 + 0.0011]))
    assert oracle.compare(ok, ref)["pass"]
    assert not oracle.compare(bad, ref)["pass"]
    # |r| in [64,128): ulp = 2^-4, two ulps pass, three fail
    ref = oracle.encode(np.array([100.0]))
    assert oracle.compare(oracle.encode(np.array([100.0 + 2 * 2.0 ** -4])), ref)["pass"]
    assert not oracle.compare(oracle.encode(np.array([100.0 + 3 * 2.0 ** -4])), ref)["pass"]
    # NaN never passes; inf against a finite value fails
    nan = np.array([0x7E00], np.uint16)
    assert not oracle.compare(nan, ref)["pass"]
    assert not oracle.compare(np.array([0x7C00], np.uint16), ref)["pass"]
    # -0 and +0 are equal
    assert oracle.compare(np.array([0x8000], np.uint16), np.array([0x0000], np.uint16))["pass"]
