"""Constructed inputs shared by the oracle pins (CPU) and the GPU parity
tests.  Only input construction lives here: no step of the method.

Double-quantization mean.  The offset is fp32(S / n) with S a float64 sum
taken in a fixed tree: sequential sums over runs of 256 scales, then over
runs of 256 partial sums, until one value remains.  The inputs below put the
exact mean right on an fp32 rounding midpoint and mix scales 2^62 times apart,
so float64 partial sums round and the order of the additions decides the
fp32 result."""
from __future__ import annotations

import numpy as np


def mean_two_level() -> np.ndarray:
    """1024 scales (4 runs of 256, two tree levels): tiny values k * 2^-38
    (k = 1..3, seeded), one 2^24 at index 462 and one 1.0 at index 511, so the
    exact mean lies just above the fp32 midpoint 16384 + 2^-10.

    With the fixed 256-run tree, run 1 sums to 2^24 + 1 and each of the other
    three run sums is just under half a float64 ulp of it (2^-29), so the
    upper level absorbs them one at a time: S = 2^24 + 1, an exact fp32 tie
    that rounds to 16384.0.  Summed sequentially over all 1024, pairwise, in
    runs of 64, 128 or 512, in runs of 256 with the upper level pairwise, or by
    numpy's pairwise np.sum, enough of the small values survive to round the
    mean up to 16384.002, which is also the correctly rounded exact mean
    (found by a seeded search over such mixtures; the pins assert each of
    these differences)."""
    rng = np.random.default_rng(1786)
    rng.integers(30, 40)                      # the search drew the exponent (38) first
    a = (np.float32(2.0 ** -38) * rng.integers(1, 4, 1024).astype(np.float32)).astype(np.float32)
    a[462] = np.float32(2.0 ** 24)
    a[511] = np.float32(1.0)
    return a


def mean_three_level() -> np.ndarray:
    """4 * 65536 scales (three tree levels, four second-level partials), all
    zero except 2^24 and 1.0 in the first partial's range and one 2^-29 at the
    start of each of the other three.  Every first- and second-level sum is
    exact, so only the top level's order matters: sequentially, each 2^-29 is
    half a float64 ulp of 2^24 + 1 and ties to even (absorbed), S = 2^24 + 1
    and the mean (2^24 + 1) / 2^18 = 64 + 2^-18 is an fp32 tie that rounds to
    64.  Pairing the top level instead keeps 2^-28 and rounds up to
    64 + 2^-17."""
    a = np.zeros(4 * 65536, np.float32)
    a[0] = np.float32(2.0 ** 24)
    a[1] = np.float32(1.0)
    for j in (1, 2, 3):
        a[65536 * j] = np.float32(2.0 ** -29)
    return a
