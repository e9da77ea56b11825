"""Pins of the CPU oracle against things other than itself: closed forms,
published table values, exact-rational brute force, invariants and library
routines.  CPU only."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.stats import norm

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def frac_nearest(x: float, a: float, table) -> int:
    """Exact-rational nearest code with the tie rule (smaller |value|, then
    lower code).  Independent of the oracle's float64 formulations."""
    if a == 0:
        n = Fraction(0)
    else:
        n = Fraction(x) / Fraction(a)
    best = None
    for c, t in enumerate(table):
        ft = Fraction(float(t))
        key = (abs(n - ft), abs(ft), c)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def bf16_all_nonneg_upto(limit_bits: int) -> np.ndarray:
    """Every non-negative bf16 bit pattern <= limit (subnormals included)."""
    return np.arange(0, limit_bits + 1, dtype=np.uint32).astype(np.uint16)


def f32(v):
    return float(np.float32(v))


# ---------------------------------------------------------------- tables
def test_nf4_table_structure():
    t = O.nf4_table().astype(np.float64)
    assert t.size == 16 and t.dtype == np.float64
    assert np.all(np.diff(t) > 0)
    assert t[0] == -1.0 and t[15] == 1.0 and t[7] == 0.0
    assert (t < 0).sum() == 7 and (t > 0).sum() == 8


def test_nf4_table_is_normal_quantiles():
    """Each nonzero entry, rescaled by the largest quantile, is the normal
    quantile of an evenly spaced probability (checked with the CDF, a
    different routine from the quantile function the oracle uses)."""
    t = O.nf4_table().astype(np.float64)
    zmax = norm.ppf(O.NF4_DELTA)
    p_pos = norm.cdf(t[8:] * zmax)
    p_neg = norm.cdf(-t[:7] * zmax)
    np.testing.assert_allclose(p_pos, np.linspace(0.5, O.NF4_DELTA, 9)[1:][::1], rtol=0, atol=2e-7)
    np.testing.assert_allclose(np.sort(p_neg), np.linspace(0.5, O.NF4_DELTA, 8)[1:], rtol=0, atol=2e-7)


def test_fp4_table_is_e2m1_over_6():
    """OCP Microscaling E2M1 magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}."""
    t = O.fp4_table()
    spec = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert t[c] == np.float32(spec[c] / 6.0)
        assert t[c + 8] == -t[c]
    assert t.view(np.uint32)[8] == 0x80000000          # code 8 is -0
    assert t.view(np.uint32)[0] == 0
    assert t.max() == 1.0 and t.min() == -1.0


def test_linear8_table_is_correctly_rounded():
    t = O.linear8_table()
    for k in range(256):
        exact = Fraction(k - 127, 127)
        v = Fraction(float(t[k]))
        up = Fraction(float(np.nextafter(t[k], np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(t[k], np.float32(-np.inf))))
        assert abs(v - exact) <= abs(up - exact) and abs(v - exact) <= abs(dn - exact)
    assert t[127] == 0 and t[0] == -1 and t[254] == 1


def test_code_tables_golden():
    """Regression guard: bit patterns written by tests/golden/make_golden.py."""
    with open(os.path.join(GOLDEN, "code_tables.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    got = {"nf4": O.nf4_table(), "fp4": O.fp4_table()}
    for name, *hexes in lines:
        assert [int(h, 16) for h in hexes] == got[name].view(np.uint32).tolist()


# ---------------------------------------------------------------- nearest code
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_nearest_matches_rational_bruteforce(qt, dtype):
    rng = np.random.default_rng(7)
    table = O.code_table(qt)
    x = rng.standard_normal(512) * rng.choice([1e-3, 0.02, 1.0, 300.0], 512)
    x = torch.from_numpy(x).to(torch.float32)
    if dtype != "fp32":
        x = x.to({"bf16": torch.bfloat16, "fp16": torch.float16}[dtype])
    x = x.to(torch.float64).numpy().reshape(16, 32)
    a = np.abs(x).max(axis=1, keepdims=True) * np.ones_like(x)
    got = O.nearest_codes(x, a, table)
    want = [frac_nearest(float(xi), float(ai), table) for xi, ai in zip(x.ravel(), a.ravel())]
    assert got.tolist() == want


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_nearest_exact_ties_go_toward_zero(qt):
    """x = a * m exactly: possible in fp32 when m's significand fits 24 bits
    and a is a power of two.  The tie must pick the smaller |value|."""
    table = O.code_table(qt)
    vals = sorted({float(v) for v in table})
    ties = 0
    for lo, hi in zip(vals[:-1], vals[1:]):
        m = Fraction(lo) + Fraction(hi)
        m /= 2
        for a in (1.0, 2.0 ** -7, 2.0 ** 9):
            x = m * Fraction(a)
            if Fraction(f32(float(x))) != x:
                continue
            ties += 1
            code = int(O.nearest_codes(np.array([float(x)]), np.array([a]), table)[0])
            want_val = lo if abs(lo) < abs(hi) else hi
            assert float(table[code]) == want_val
            assert code == frac_nearest(float(x), a, table)
    assert ties > 0


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_nearest_exhaustive_bf16_sweep(qt):
    """All bf16 |x| <= a for a sample of bf16 absmax mantissas in [1, 2), both
    signs: the two float64 formulations agree (asserted inside the oracle) and
    the 150 pairs closest to a midpoint match exact rational search."""
    table = O.code_table(qt)
    vals = sorted({float(v) for v in table})
    mids = np.array([(l + h) / 2 for l, h in zip(vals[:-1], vals[1:])])
    for mant in (0, 1, 37, 85, 127):
        abits = 0x3F80 | mant
        a = float(O.bf16_bits_to_f64(np.array([abits], np.uint16))[0])
        pos = O.bf16_bits_to_f64(bf16_all_nonneg_upto(abits))
        x = np.concatenate([pos, -pos])
        codes = O.nearest_codes(x, np.full_like(x, a), table)
        n = x / a
        dist = np.min(np.abs(n[:, None] - mids[None, :]), axis=1)
        near = np.argsort(dist, kind="stable")[:150]       # the hardest pairs
        for i in near:
            assert codes[i] == frac_nearest(float(x[i]), a, table)
        # monotone: codes, read as values, never decrease with x
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(table[codes[order]].astype(np.float64)) >= 0)


def test_fp4_bf16_decisions_equal_real_e2m1_rounding():
    """For bf16 data the fp32-table decision equals rounding x/a to the nearest
    real E2M1/6 value with ties toward zero, even at ratios such as 1/8 that
    sit exactly on a real midpoint (k/24) and a few 1e-9 below the fp32 one."""
    table = O.fp4_table()
    real = [Fraction(v, 12) for v in (0, 1, 2, 3, 4, 6, 8, 12)]
    real = [-v for v in real[:0:-1]] + real                 # ascending, one zero
    checked = on_mid = 0
    for mant in (0, 5, 64, 100, 127):
        abits = 0x3F80 | mant
        a = float(O.bf16_bits_to_f64(np.array([abits], np.uint16))[0])
        pos = O.bf16_bits_to_f64(bf16_all_nonneg_upto(abits))
        x = np.concatenate([pos, -pos])
        codes = O.nearest_codes(x, np.full_like(x, a), table)
        r24 = np.abs(x / a * 24 - np.round(x / a * 24))
        cand = np.flatnonzero(r24 < 1e-3)
        exact_mid = cand[np.round(x[cand] / a * 24) % 2 == 1]        # on a real midpoint
        for i in np.concatenate([exact_mid[:200], cand[::max(1, cand.size // 300)]]):
            n = Fraction(float(x[i])) / Fraction(a)
            best = min(real, key=lambda v: (abs(n - v), abs(v)))
            on_mid += int(sum(abs(n - v) == abs(n - best) for v in real) > 1)
            assert Fraction(float(table[codes[i]])) == Fraction(float(np.float32(float(best))))
            checked += 1
    assert checked > 1000 and on_mid > 10


def test_lut_snapping_is_not_exact():
    """The CPU failure mode the PR page documents: snapping the normalised
    value to a 65536-point grid before the 8-bit codebook lookup misses some
    values that exact search gets right.  The oracle is the exact one."""
    rng = np.random.default_rng(11)
    code = O.linear8_table()
    x = torch.from_numpy(rng.standard_normal(1 << 20)).to(torch.float32).to(torch.float64).numpy()
    x = x.reshape(-1, 256)
    a = np.abs(x).max(axis=1, keepdims=True) * np.ones_like(x)
    exact = O.nearest_codes(x.ravel(), a.ravel(), code)
    grid = np.round((x / a + 1.0) * 32767.5) / 32767.5 - 1.0
    snapped = O.nearest_codes_literal(grid.ravel(), np.ones(grid.size), code)
    bad = np.flatnonzero(snapped != exact)
    assert bad.size > 0
    for i in bad[:50]:
        assert exact[i] == frac_nearest(float(x.ravel()[i]), float(a.ravel()[i]), code)


# ---------------------------------------------------------------- quantize
def test_absmax_element_roundtrips_and_zero_code():
    for qt in ("nf4", "fp4"):
        x = np.array([0.5, -0.25, 0.0, -0.0, 1e-30, -2.0, 2.0 ** -20, 0.125] * 8)
        packed, absmax = O.quantize_4bit(x, 64, qt)
        codes = O.unpack_nibbles(packed, x.size)
        t = O.code_table(qt)
        assert absmax.tolist() == [2.0]
        zero = int(np.flatnonzero(t == 0)[0])
        assert codes[2] == zero and codes[3] == zero        # +0 and -0 -> lowest zero code
        assert t[codes[5]] == -1.0
        w = O.dequantize_4bit(packed, absmax, x.size, 64, qt)
        assert w[5] == -2.0


def test_zero_block_and_partial_block():
    x = np.concatenate([np.zeros(64), np.linspace(-1, 1, 37)])      # 101 elements
    packed, absmax = O.quantize_4bit(x, 64, "nf4")
    assert packed.size == 51 and absmax.size == 2
    assert absmax[0] == 0.0 and absmax[1] == 1.0
    codes = O.unpack_nibbles(packed, 101)
    assert np.all(codes[:64] == 7)
    assert packed[-1] & 15 == 0                       # odd tail: low nibble empty
    w = O.dequantize_4bit(packed, absmax, 101, 64, "nf4")
    assert np.all(w[:64].view(np.uint32) == 0)


def test_pack_order_high_nibble_first():
    """Reading R4 (nibble order; parity unpinned against external data)."""
    assert O.pack_nibbles([3, 12]).tolist() == [0x3C]
    assert O.pack_nibbles([9]).tolist() == [0x90]
    assert O.unpack_nibbles(np.array([0xA5], np.uint8), 2).tolist() == [10, 5]


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_reconstruction_error_at_most_half_gap(qt):
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal(64 * 200) * 0.02).to(torch.bfloat16)
    x = x.to(torch.float64).numpy()
    packed, absmax = O.quantize_4bit(x, 64, qt)
    w = O.dequantize_4bit(packed, absmax, x.size, 64, qt).astype(np.float64)
    a = np.repeat(absmax.astype(np.float64), 64)
    vals = np.array(sorted({float(v) for v in O.code_table(qt)}))
    n = x / a
    j = np.clip(np.searchsorted(vals, n) - 1, 0, vals.size - 2)   # bracketing pair
    half_gap = (vals[j + 1] - vals[j]) / 2 * a
    ulp = np.spacing(np.abs(w).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(x - w) <= half_gap + ulp)


# ---------------------------------------------------------------- double quant
def test_mean_tree_within_one_ulp_of_exact_mean():
    rng = np.random.default_rng(5)
    for n in (1, 7, 256, 257, 70000):
        a = np.abs(rng.standard_normal(n)).astype(np.float32) * np.float32(0.05)
        off = O.mean_fixed_tree(a)
        exact = sum(Fraction(float(v)) for v in a) / n
        ulp = Fraction(float(np.spacing(np.float32(abs(float(exact))))))
        assert abs(Fraction(float(off)) - exact) <= ulp


def test_double_quant_codes_exact_and_bounded():
    rng = np.random.default_rng(9)
    a = (np.abs(rng.standard_normal(1000)) * 0.03).astype(np.float32)
    a[300:556] = a[300]                       # a group of equal scales
    q, s, off = O.double_quant(a, 256)
    assert q.dtype == np.uint8 and s.size == 4 and s.dtype == np.float32
    code = O.linear8_table()
    c = (a - off).astype(np.float32)
    for i in range(0, 1000, 7):
        g = i // 256
        assert q[i] == frac_nearest(float(c[i]), float(s[g]), code)
    ahat = O.dequant_absmax(q, s, off, None, 256)
    bound = np.repeat(s.astype(np.float64), 256)[:1000] / 254 + 2 * np.spacing(a).astype(np.float64)
    assert np.all(np.abs(ahat.astype(np.float64) - a) <= bound)


def test_double_quant_zero_group_gets_zero_code():
    a = np.full(300, 0.5, np.float32)        # every c_i is 0 -> s_g = 0
    q, s, off = O.double_quant(a, 256)
    assert off == np.float32(0.5) and np.all(s == 0) and np.all(q == 127)
    assert np.all(O.dequant_absmax(q, s, off) == np.float32(0.5))


def test_dequant_absmax_two_roundings():
    """fp32(fp32(c*s) + off), which differs from a fused multiply-add."""
    code = O.linear8_table()
    q = np.array([200], np.uint8)
    s = np.array([np.float32(0.3)], np.float32)
    off = np.float32(0.1)
    got = O.dequant_absmax(q, s, off)[0]
    p = Fraction(float(code[200])) * Fraction(float(s[0]))
    p32 = Fraction(f32(float(p)))
    assert Fraction(float(got)) == Fraction(f32(float(p32 + Fraction(float(off)))))


def test_storage_bits_per_weight():
    """4-bit codes are a quarter of fp16 ("Memory Savings" table: 7B params
    -> 3.5 GB); fp32 absmax at block 64 adds 0.5 bit; double quantization
    brings the scales to 8 bits plus one fp32 per 256 blocks."""
    numel = 4096 * 64
    x = np.linspace(-1, 1, numel).astype(np.float32).astype(np.float64)
    packed, absmax = O.quantize_4bit(x, 64, "nf4")
    assert packed.size * 8 / numel == 4.0
    assert (packed.size + 4 * absmax.size) * 8 / numel == 4.5
    q, s, off = O.double_quant(absmax, 256)
    bits = (packed.size + q.size + 4 * s.size) * 8 / numel
    assert abs(bits - 4.127) < 1e-3
    with open(os.path.join(GOLDEN, "memory_savings.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for params, fp16_gb, q4_gb in rows:
        n = float(params) * 1e9
        assert n * 2 / 1e9 == pytest.approx(float(fp16_gb))
        assert n * packed.size / numel / 1e9 == pytest.approx(float(q4_gb))


# ---------------------------------------------------------------- dequantize
def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(37.0)
    u = x.view(np.uint32)
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000      # exact halfway cases
    x = u.view(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), want)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_dequantize_is_one_fp32_rounding(qt):
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, 64 * 50).astype(np.uint8)
    absmax = (np.abs(rng.standard_normal(50)) * 0.07).astype(np.float32)
    packed = O.pack_nibbles(codes)
    w = O.dequantize_4bit(packed, absmax, codes.size, 64, qt)
    want = O.code_table(qt)[codes] * np.repeat(absmax, 64)    # numpy fp32 multiply
    assert np.array_equal(w.view(np.uint32), want.astype(np.float32).view(np.uint32))
    wb = O.dequantize_4bit(packed, absmax, codes.size, 64, qt, "bf16")
    tb = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(wb, tb.view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------- matmuls
def _small_state(N=24, K=128, bs=32, qt="nf4", seed=4):
    rng = np.random.default_rng(seed)
    W = torch.from_numpy(rng.standard_normal((N, K)) * 0.02).to(torch.bfloat16)
    W = W.to(torch.float64).numpy()
    packed, absmax = O.quantize_4bit(W, bs, qt)
    return W, packed, absmax


def test_gemv_one_hot_returns_column_exactly():
    N, K, bs = 24, 128, 32
    _, packed, absmax = _small_state(N, K, bs)
    What = O.dequantize_4bit(packed, absmax, N * K, bs).reshape(N, K)
    for k in (0, 5, 127):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        y = O.matmul_4bit(x, packed, absmax, N, K, bs)
        assert np.array_equal(y[0], What[:, k].astype(np.float64))


def test_gemm_bruteforce_fsum_small():
    N, K, bs = 24, 128, 32
    _, packed, absmax = _small_state(N, K, bs, "fp4")
    rng = np.random.default_rng(6)
    X = rng.standard_normal((3, K))
    Y = O.matmul_4bit(X, packed, absmax, N, K, bs, "fp4")
    codes = O.unpack_nibbles(packed, N * K).reshape(N, K)
    t = O.fp4_table()
    for m in range(3):
        for n in range(N):
            terms = [X[m, k] * float(np.float32(t[codes[n, k]] * absmax[(n * K + k) // bs]))
                     for k in range(K)]
            assert Y[m, n] == pytest.approx(math.fsum(terms), rel=1e-12, abs=1e-15)
    rows = [3, 0, 17]
    np.testing.assert_allclose(
        O.matmul_4bit_rows(X, packed, absmax, N, K, bs, "fp4", rows), Y[:, rows],
        rtol=1e-13, atol=1e-16)


def test_backward_is_the_adjoint_of_the_forward():
    """<dY, X W^T> = <dY W, X> for any X and dY (the backward of y = x W^T
    with respect to x), and a one-hot dY row returns that weight row exactly:
    a transposed or mis-indexed weight fails one of the two."""
    N, K, bs = 24, 128, 32
    _, packed, absmax = _small_state(N, K, bs, "nf4", seed=9)
    rng = np.random.default_rng(10)
    X = rng.standard_normal((5, K))
    dY = rng.standard_normal((5, N))
    Y = O.matmul_4bit(X, packed, absmax, N, K, bs)
    dX = O.matmul_4bit_backward(dY, packed, absmax, N, K, bs)
    assert dX.shape == (5, K)
    lhs = math.fsum((dY * Y).ravel())
    rhs = math.fsum((dX * X).ravel())
    assert lhs == pytest.approx(rhs, rel=1e-12, abs=1e-14)
    What = O.dequantize_4bit(packed, absmax, N * K, bs).reshape(N, K)
    for n in (0, 7, 23):
        e = np.zeros((1, N))
        e[0, n] = 1.0
        assert np.array_equal(O.matmul_4bit_backward(e, packed, absmax, N, K, bs)[0],
                              What[n].astype(np.float64))


def test_quantize_full_pipeline_small_bf16_roundtrip():
    """dequant(quant(x)) stays within the code gaps for DQ'd scales too."""
    rng = np.random.default_rng(8)
    W = torch.from_numpy(rng.standard_normal(128 * 64) * 0.02).to(torch.bfloat16)
    W = W.to(torch.float64).numpy()
    packed, absmax = O.quantize_4bit(W, 64, "nf4")
    q, s, off = O.double_quant(absmax, 256)
    ahat = O.dequant_absmax(q, s, off)
    w = O.dequantize_4bit(packed, ahat, W.size, 64, "nf4").astype(np.float64)
    rel = np.linalg.norm(w - W) / np.linalg.norm(W)
    assert rel < 0.12


# ---------------------------------------------------------------- 8-bit blockwise codec
def _f32_nearest(q: Fraction) -> float:
    """Correctly rounded fp32 of an exact rational (round to nearest even)."""
    v = np.float32(float(q))
    best = None
    for c in (np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, float(c))
    return best[1]


def _decode_tree_byte(b: int) -> Fraction:
    """Decode one byte of the dynamic-tree layout from its bits: sign, then a
    run of e zero bits (the decimal exponent), a one bit, then 6 - e fraction
    bits j selecting the centre of bin j of [0.1, 1] cut into 2^(6-e) bins.
    The all-zero magnitude stands for 0 (positive sign) or 1 (negative sign)."""
    sign, mag = b >> 7, b & 0x7F
    if mag == 0:
        return Fraction(1) if sign else Fraction(0)
    e = 7 - mag.bit_length()            # leading zero bits of the 7-bit field
    nf = 6 - e
    j = mag & ((1 << nf) - 1)
    centre = Fraction(1, 10) + Fraction(9, 10) * Fraction(2 * j + 1, 2 ** (nf + 1))
    v = centre / Fraction(10) ** e
    return -v if sign else v


def test_dynamic_tree_table_from_bit_layout():
    """Every byte decoded from the bit layout, rounded once to fp32, gives the
    oracle's sorted table exactly; decades hold 64, 32, ..., 1 values."""
    t = O.dynamic_tree_table()
    want = sorted(_f32_nearest(_decode_tree_byte(b)) for b in range(256))
    assert t.dtype == np.float32 and t.size == 256
    assert t.tolist() == want
    assert np.all(np.diff(t) > 0)
    pos = t[t > 0]
    assert pos.max() == 1.0 and np.array_equal(np.sort(-t[t < 0]), pos[pos < 1])
    for e in range(7):
        lo, hi = 0.1 * 10.0 ** -e, 10.0 ** -e
        assert int(((pos > lo) & (pos < hi)).sum()) == 2 ** (6 - e)


def _frac_table(table):
    return [Fraction(float(v)) for v in table]


def _frac_nearest_fast(x: float, a: float, ftab) -> int:
    n = Fraction(0) if a == 0 else Fraction(x) / Fraction(a)
    return min(range(len(ftab)), key=lambda c: (abs(n - ftab[c]), abs(ftab[c]), c))


@pytest.mark.parametrize("table", ["linear", "dynamic"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_blockwise_codes_match_rational_bruteforce(table, dtype):
    rng = np.random.default_rng(21)
    n, bs = 600, 128                      # four full blocks and a ragged one
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    x = torch.from_numpy(rng.standard_normal(n) * np.repeat(10.0 ** rng.uniform(-3, 1, 5), bs)[:n])
    x = x.to(tdt).to(torch.float64).numpy()
    x[130:140] = 0.0                       # zeros inside a live block
    code = O.linear8_table() if table == "linear" else O.dynamic_tree_table()
    q, absmax = O.quantize_blockwise(x, bs, code)
    assert q.dtype == np.uint8 and absmax.dtype == np.float32 and absmax.size == 5
    for b in range(5):
        assert float(absmax[b]) == float(np.max(np.abs(x[b * bs:(b + 1) * bs])))
    ftab = _frac_table(code)
    want = [_frac_nearest_fast(float(x[i]), float(absmax[i // bs]), ftab) for i in range(n)]
    assert q.tolist() == want


def test_blockwise_exact_ties_and_extremes():
    """Midpoints of adjacent dynamic-tree values, scaled by an exact power of
    two, sit exactly on the tie and go to the smaller magnitude; the block's
    largest positive element takes the code of 1."""
    t = O.dynamic_tree_table()
    mids = (t[:-1].astype(np.float64) + t[1:].astype(np.float64)) / 2.0
    a = 4.0
    x = np.concatenate([[a], mids * a])          # first element fixes absmax = a
    q, absmax = O.quantize_blockwise(x, x.size, t)
    assert absmax.tolist() == [a] and t[q[0]] == 1.0
    for k in range(mids.size):
        lo, hi = k, k + 1
        assert q[k + 1] == (lo if abs(t[lo]) < abs(t[hi]) else hi)


def test_blockwise_zero_block_and_roundtrip_bound():
    rng = np.random.default_rng(5)
    bs = 256
    x = rng.standard_normal(bs * 6 + 77) * 0.3
    x[bs:2 * bs] = 0.0
    for code in (O.linear8_table(), O.dynamic_tree_table()):
        q, absmax = O.quantize_blockwise(x, bs, code)
        zero = int(np.flatnonzero(code == 0)[0])
        assert absmax[1] == 0 and np.all(q[bs:2 * bs] == zero)
        w = O.dequantize_blockwise(q, absmax, bs, code)
        assert w.dtype == np.float32 and np.all(w[bs:2 * bs] == 0)
        # |x / absmax| <= 1, so the error is at most absmax times the larger of
        # half the widest gap and the distance from +-1 to the table's ends,
        # plus the final fp32 rounding of w
        c64 = code.astype(np.float64)
        reach = max(np.max(np.diff(c64)) / 2, 1 - c64.max(), 1 + c64.min())
        a_el = np.repeat(absmax.astype(np.float64), bs)[: x.size]
        assert np.all(np.abs(w - x) <= reach * a_el + np.abs(w) * 2.0 ** -24)


def test_dequantize_blockwise_is_one_fp32_rounding():
    rng = np.random.default_rng(8)
    bs = 64
    q = rng.integers(0, 256, bs * 30 + 9).astype(np.uint8)
    absmax = (np.abs(rng.standard_normal(31)) * 3.0).astype(np.float32)
    t = O.dynamic_tree_table()
    w = O.dequantize_blockwise(q, absmax, bs, t)
    for i in range(0, q.size, 7):
        exact = Fraction(float(t[q[i]])) * Fraction(float(absmax[i // bs]))
        assert float(w[i]) == _f32_nearest(exact)
    wb = O.dequantize_blockwise(q, absmax, bs, t, "bf16")
    tb = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wb, tb)
    wh = O.dequantize_blockwise(q, absmax, bs, t, "fp16")
    assert np.array_equal(np.asarray(wh).view(np.uint16), w.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------- embedding
def test_embedding_is_a_one_hot_product():
    """Gathering rows equals multiplying a one-hot matrix by the dequantized
    table (the backward's dY @ W_hat): every product is 0 or 1 times a
    weight, so the float64 sums are exact.  Out-of-range indices are all-zero
    one-hot rows."""
    rng = np.random.default_rng(14)
    V, D, bs = 40, 128, 64
    W = torch.from_numpy(rng.standard_normal((V, D)) * 0.05).to(torch.bfloat16).to(torch.float64).numpy()
    packed, absmax = O.quantize_4bit(W, bs, "nf4")
    idx = np.array([0, 39, 7, 7, -1, 40, 13, 1000, 22])
    got = O.embedding_4bit(idx, packed, absmax, V, D, bs, "nf4")
    onehot = np.zeros((idx.size, V))
    for t, i in enumerate(idx):
        if 0 <= i < V:
            onehot[t, i] = 1.0
    want = O.matmul_4bit_backward(onehot, packed, absmax, V, D, bs, "nf4")
    assert np.array_equal(got.astype(np.float64), want)
    assert not got[4].any() and not got[5].any() and not got[7].any()


def test_embedding_rows_by_hand_odd_width():
    """D = 45 (odd): rows start in the middle of a byte and blocks straddle
    rows; each element is decoded by hand from its byte, nibble and block."""
    rng = np.random.default_rng(15)
    V, D, bs = 11, 45, 32
    W = (rng.standard_normal(V * D) * 0.1).astype(np.float32).astype(np.float64)
    for qt in ("nf4", "fp4"):
        packed, absmax = O.quantize_4bit(W, bs, qt)
        t = O.code_table(qt)
        idx = np.array([3, 0, 10, 3])
        got = O.embedding_4bit(idx, packed, absmax, V, D, bs, qt)
        for r, i in enumerate(idx):
            for d in range(D):
                e = i * D + d
                byte = int(packed[e // 2])
                code = byte >> 4 if e % 2 == 0 else byte & 15
                assert got[r, d] == np.float32(t[code] * np.float32(absmax[e // bs]))
