"""Pins of the oracle's two rounding-order definitions against exact-rational
re-derivations written here (CPU only):

* fp32 -> fp16 conversion (the output rounding of dequantize_4bit and of the
  8-bit codec for fp16): round to nearest, ties to even, subnormals included,
  checked against an exact-rational rounding of the fp32 value and against
  torch's conversion, on constructed halfway cases and random values.
* the double-quantization mean ("mps-bitsandbytes 0.4.7", "Functional API",
  double_quant): fp32(S / n) with S the float64 sum in the fixed tree of
  sequential runs of 256.  Every float64 addition is re-done here as an exact
  rational sum rounded once to float64, the tree is walked recursively, and
  crafted inputs make every plausible other order (flat, pairwise, other
  fan-ins, a pairwise upper level, numpy's np.sum) give a different fp32
  offset, so a wrong order in the oracle fails."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from crafted_inputs import mean_three_level, mean_two_level


# ---------------------------------------------------------------- exact rounding
def _floor_log2(m: Fraction) -> int:
    e = m.numerator.bit_length() - m.denominator.bit_length()
    while Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    return e


def rne_binary(v: Fraction, p: int, emin: int) -> Fraction:
    """Round an exact rational to the nearest value with p significant bits
    whose exponent is at least emin (gradual underflow below 2^emin), ties to
    the even significand.  No overflow handling: callers stay in range."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    m = abs(v)
    e = max(_floor_log2(m), emin)
    q = Fraction(2) ** (e - (p - 1))          # spacing of the binade (or subnormals)
    k = m / q
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def f64_add(x: float, y: float) -> float:
    """float64 addition as an exact rational sum rounded once (RNE)."""
    r = rne_binary(Fraction(x) + Fraction(y), 53, -1022)
    return r.numerator / r.denominator        # exact: r is a float64 value


def f64_div(x: float, n: int) -> float:
    r = rne_binary(Fraction(x) / n, 53, -1022)
    return r.numerator / r.denominator


def to_f32(x: float) -> float:
    r = rne_binary(Fraction(x), 24, -126)
    return r.numerator / r.denominator


# ---------------------------------------------------------------- fp16
FP16_P, FP16_EMIN = 11, -14


def _fp16_grid_cases():
    """fp32 values on and next to fp16 rounding midpoints: normal binades,
    the subnormal range, the subnormal/normal boundary and the top binade."""
    out = []
    for e in (-14, -13, -9, -1, 0, 3, 10, 15):           # normal binades 2^e
        q = Fraction(2) ** (e - 10)
        for k in (1024, 1025, 1100, 1537, 2046, 2047):   # even and odd significands
            if e == 15 and k > 2046:
                continue                                  # midpoint above 65504: overflow
            mid = (k + Fraction(1, 2)) * q
            out.append(mid)
    for k in (0, 1, 2, 3, 100, 511, 1022, 1023):          # subnormals: spacing 2^-24
        out.append((k + Fraction(1, 2)) * Fraction(2) ** -24)
    vals = []
    for mid in out:
        m32 = np.float32(float(mid))
        assert Fraction(float(m32)) == mid               # every midpoint is an fp32 value
        for v in (np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(np.inf))):
            vals += [v, -v]
    vals += [np.float32(65504.0), np.float32(65519.99), np.float32(2.0 ** -24),
             np.float32(2.0 ** -14), np.float32(0.0), np.float32(-0.0), np.float32(1e-30)]
    return np.array(vals, dtype=np.float32)


def test_f32_to_f16_constructed_halfway_and_subnormal_cases():
    x = _fp16_grid_cases()
    got = O.f32_to_f16(x)
    for v, g in zip(x, got):
        want = rne_binary(Fraction(float(v)), FP16_P, FP16_EMIN)
        assert Fraction(float(g)) == want, (float(v), float(g), float(want))
    # the halfway cases really are ties that go to the even neighbour
    assert float(O.f32_to_f16(np.float32(2.0 ** -25))[()]) == 0.0
    assert float(O.f32_to_f16(np.float32(3 * 2.0 ** -25))[()]) == 2.0 ** -23
    assert float(O.f32_to_f16(np.float32(1 + 2.0 ** -11))[()]) == 1.0
    assert float(O.f32_to_f16(np.float32(1 + 3 * 2.0 ** -11))[()]) == 1 + 2.0 ** -9


def test_f32_to_f16_random_against_rational_and_torch():
    rng = np.random.default_rng(31)
    mag = 2.0 ** rng.uniform(-26, 15.99, 4000)
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    got = O.f32_to_f16(x)
    for v, g in zip(x[:1500], got[:1500]):
        assert Fraction(float(g)) == rne_binary(Fraction(float(v)), FP16_P, FP16_EMIN)
    ref = torch.from_numpy(x).to(torch.float16).numpy()
    assert np.array_equal(np.asarray(got).view(np.uint16), ref.view(np.uint16))


# ---------------------------------------------------------------- mean tree
def tree_mean_rational(a, fanin=256) -> float:
    """The fixed tree walked recursively: a level's runs of ``fanin`` are
    summed left to right with exactly rounded float64 additions; then
    fp32(f64(S / n))."""
    vals = [float(v) for v in np.asarray(a, dtype=np.float32)]

    def level_sums(level):
        sums = []
        for i in range(0, len(level), fanin):
            acc = 0.0
            for j, v in enumerate(level[i:i + fanin]):
                acc = v if j == 0 else f64_add(acc, v)
            sums.append(acc)
        return sums

    level = vals
    while len(level) > 1:
        level = level_sums(level)
    return to_f32(f64_div(level[0], len(vals)))


def _flat(a):
    s = 0.0
    for v in a:
        s += float(v)
    return s


def _pairwise(vals):
    v = [float(x) for x in vals]
    while len(v) > 1:
        if len(v) % 2:
            v.append(0.0)
        v = [v[i] + v[i + 1] for i in range(0, len(v), 2)]
    return v[0]


def _tree(a, fanin, upper_pairwise=False):
    level = [float(v) for v in a]
    first = True
    while len(level) > 1:
        if upper_pairwise and not first:
            return _pairwise(level)
        level = [_flat(level[i:i + fanin]) for i in range(0, len(level), fanin)]
        first = False
    return level[0]


def _f32_mean(S, n):
    return float(np.float32(S / n))


@pytest.mark.parametrize("n", [1, 2, 255, 256, 257, 513, 65536, 65537, 70000])
def test_mean_tree_matches_rational_walk(n):
    rng = np.random.default_rng(n)
    a = (np.abs(rng.standard_normal(n)) * 0.05).astype(np.float32)
    a[:: 37] *= np.float32(1e6)                       # wide exponents: sums do round
    assert float(O.mean_fixed_tree(a)) == tree_mean_rational(a)


def test_mean_tree_crafted_order_two_levels():
    a = mean_two_level()
    n = a.size
    got = float(O.mean_fixed_tree(a))
    assert got == tree_mean_rational(a) == 16384.0
    others = {
        "flat": _flat(a), "pairwise": _pairwise(a), "runs of 64": _tree(a, 64),
        "runs of 128": _tree(a, 128), "runs of 512": _tree(a, 512),
        "runs of 256, pairwise above": _tree(a, 256, upper_pairwise=True),
        "np.sum": float(np.sum(a.astype(np.float64))),
    }
    for name, S in others.items():
        assert _f32_mean(S, n) != got, f"{name} gives the same offset: the input has no teeth"
    # the exact mean rounds the other way: the tree order, not exactness, fixes the bits
    exact = sum(Fraction(float(v)) for v in a) / n
    assert to_f32(float(exact)) != got


def test_mean_tree_crafted_order_top_level():
    a = mean_three_level()
    got = float(O.mean_fixed_tree(a))
    assert got == tree_mean_rational(a) == 64.0
    assert _f32_mean(_tree(a, 256, upper_pairwise=True), a.size) == 64.0 + 2.0 ** -17
    lvl2 = [_tree(a[i:i + 65536], 256) for i in range(0, a.size, 65536)]
    assert _f32_mean((lvl2[0] + lvl2[1]) + (lvl2[2] + lvl2[3]), a.size) != got
