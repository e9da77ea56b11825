"""Plain CPU oracle: 4-bit blockwise quantization (NF4 / FP4), double-quantized
absmax, dequantization and the dequantize-then-multiply (gemv / gemm and the
gemm input gradient).

TEST INFRASTRUCTURE ONLY.  This module exists to check the GPU library.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run it; the product library neither imports it nor
shares a kernel, table, helper or constant generator with it.

Everything is numpy float64 or exact rationals, written to be read against the
pages, not to be fast.  Citations name the web page by its title and the
section the statement sits in:

* "Feat/mps gemm 4bit bf16" (a pull request page), sections "What runs
  natively now" (the op set: quantize_4bit / dequantize_4bit, gemv_4bit as a
  fused dequant+dot, gemm_4bit as dequant then GEMM; unsupported blocksize and
  K % 32 guards), "Correctness" (bit-exact codec, matmuls within per-dtype
  tolerance) and "Known failures" (an exact float64 nearest-code search is the
  reference; snapping the normalised value to a 65536-point table first is the
  documented source of CPU mismatches).
* "mps-bitsandbytes 0.4.7" (a package page), sections "Features" (NF4 for
  normally distributed LLM weights, FP4, double quantization of the scales),
  "Functional API" (``quantize_nf4(tensor, block_size=64)`` returning packed
  codes and per-block absmax; ``double_quant(absmax, double_quant_block=256)``
  and ``dequant_absmax``), "Memory Savings" (4-bit = a quarter of fp16) and
  "Credits" (NF4 comes from the QLoRA paper).

Readings taken where the pages are silent (the same list is kept with the
design notes):

R1  NF4 table: the QLoRA quantile construction in float64 with
    delta = 0.9677083, 8 positive and 7 negative normal quantiles plus an exact
    zero, normalised by the largest, rounded once to fp32; code = ascending rank.
R2  FP4 table: OCP E2M1 (code bits s e1 e0 m) divided by 6 so the largest
    magnitude is 1; codes 0-7 positive, 8-15 negative (code 8 is -0).
R3  Nearest code: exact argmin of |x/a - T[c]| over the fp32 table values.  An
    exact tie goes to the smaller |T[c]|; among equal values the lower code
    wins (so every value that rounds to zero gets the lowest zero code).
    A block whose absmax is 0 encodes every element with that zero code.
R4  Packing: byte j = (code[2j] << 4) | code[2j+1]; an odd tail leaves the low
    nibble 0.  Blocks are runs of ``blocksize`` elements of the row-major
    flattening; the last block may be partial.
R5  Double quantization: offset = fp32(S / nblocks) where S is a float64 sum in
    a fixed tree (sequential sums over runs of 256, repeated until one value);
    c_i = fp32(a_i - offset); per group of ``blocksize2`` scales s_g = max|c_i|;
    q_i = nearest code of c_i / s_g in an 8-bit table (default: the fp32
    quotients (k - 127) / 127), same rule as R3.
R6  Scale reconstruction: a_hat = fp32(fp32(code2[q] * s_g) + offset) -- two
    roundings, no fused multiply-add.
R7  Dequantize: w = fp32(T[code] * a_hat) (the float64 product is exact), then
    round-to-nearest-even into bf16 or fp16 when asked.
R8  gemv / gemm: Y = X @ W_hat^T with W_hat the fp32 dequantized weight of R7,
    computed in float64 -- the pages' own fallback composition (dequantize,
    then a linear layer).

Parity status: every function below is pinned by ``tests/test_oracle_*.py``
against closed forms, published table values, exact-rational brute force or
invariants.  Two readings have no external data to pin against and are marked
"parity unpinned" where they are used: R4's nibble order and the exact fp32
bits of R1 against other libraries' NF4 tables.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
from scipy.stats import norm

__all__ = [
    "NF4_DELTA", "MEAN_FANIN", "nf4_table", "fp4_table", "code_table",
    "linear8_table", "bf16_bits_to_f64", "f32_to_bf16_bits", "f32_to_f16",
    "block_absmax", "nearest_codes", "nearest_codes_literal",
    "nearest_codes_threshold", "pack_nibbles", "unpack_nibbles",
    "quantize_4bit", "mean_fixed_tree", "double_quant", "dequant_absmax",
    "dequantize_4bit", "dequantize_rows", "matmul_4bit", "matmul_4bit_rows",
    "matmul_4bit_backward", "dynamic_tree_table", "quantize_blockwise",
    "dequantize_blockwise", "embedding_4bit",
]

NF4_DELTA = 0.9677083      # R1
MEAN_FANIN = 256           # R5: fan-in of the fixed summation tree
_CHUNK = 1 << 18           # elements per vectorised chunk (memory bound only)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x32) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite input)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_to_f16(x32) -> np.ndarray:
    """fp32 -> fp16, round to nearest even (numpy's conversion is IEEE)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------
# code tables (R1, R2, R5)
# --------------------------------------------------------------------------
def nf4_table() -> np.ndarray:
    """NF4 values, ascending (R1).  "Features": NF4 targets normally
    distributed weights; "Credits": the construction is QLoRA's."""
    pos = norm.ppf(np.linspace(NF4_DELTA, 0.5, 9)[:-1])     # 8 positive quantiles
    neg = -norm.ppf(np.linspace(NF4_DELTA, 0.5, 8)[:-1])    # 7 negative quantiles
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    return (v / v.max()).astype(np.float32)


def fp4_table() -> np.ndarray:
    """FP4 values by code (R2): E2M1 decoded from its bit fields, divided by 6."""
    out = np.empty(16, dtype=np.float32)
    for c in range(16):
        sign, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
        out[c] = np.float32((-1.0 if sign else 1.0) * mag / 6.0)
    return out


def code_table(quant_type: str) -> np.ndarray:
    if quant_type == "nf4":
        return nf4_table()
    if quant_type == "fp4":
        return fp4_table()
    raise ValueError(f"unknown quant_type {quant_type!r}")


def linear8_table() -> np.ndarray:
    """Default second-level table for double quantization (R5): the correctly
    rounded fp32 quotient (k - 127) / 127 for k = 0..255."""
    k = np.arange(256, dtype=np.float32)
    return (k - np.float32(127)) / np.float32(127)


# --------------------------------------------------------------------------
# blockwise absmax and nearest code (R3)
# --------------------------------------------------------------------------
def block_absmax(x, blocksize: int) -> np.ndarray:
    """Per block of ``blocksize`` consecutive elements, max |x| (float64, exact).
    "Functional API": quantize_nf4 returns per-block absmax scales."""
    x = np.asarray(x, dtype=np.float64).ravel()
    nb = -(-x.size // blocksize)
    pad = np.zeros(nb * blocksize, dtype=np.float64)
    pad[: x.size] = np.abs(x)
    return pad.reshape(nb, blocksize).max(axis=1)


def _sig_bits(v: float) -> int:
    """Significant bits of a finite binary float (0 for zero)."""
    f = Fraction(v)
    p = abs(f.numerator)
    if p == 0:
        return 0
    while p % 2 == 0:
        p //= 2
    return p.bit_length()


def nearest_codes_literal(x, a, table) -> np.ndarray:
    """R3 as written: n = x / a in float64 (n = 0 when a = 0), argmin over the
    table of |n - T[c]|; ties to the smaller |T[c]|, then to the lower code."""
    t = np.asarray(table, dtype=np.float32).astype(np.float64)
    pref = sorted(range(t.size), key=lambda c: (abs(t[c]), c))
    pref_rank = np.empty(t.size, dtype=np.int64)
    pref_rank[pref] = np.arange(t.size)
    x = np.asarray(x, dtype=np.float64)
    a = np.broadcast_to(np.asarray(a, dtype=np.float64), x.shape).ravel()
    x = x.ravel()
    out = np.empty(x.size, dtype=np.int64)
    step = max(1, _CHUNK * 16 // t.size)
    for s in range(0, x.size, step):
        xs, as_ = x[s:s + step], a[s:s + step]
        safe = np.where(as_ > 0, as_, 1.0)
        n = np.where(as_ > 0, xs / safe, 0.0)
        d = np.abs(n[:, None] - t[None, :])
        cand = d == d.min(axis=1, keepdims=True)
        out[s:s + step] = np.where(cand, pref_rank[None, :], t.size).argmin(axis=1)
    return out


def nearest_codes_threshold(x, a, table) -> np.ndarray:
    """R3 in threshold form: code = rank of x among the products a * m_j, m_j the
    midpoints of adjacent distinct table values.  x sits above a positive
    threshold only when strictly greater (the tie goes toward zero) and above a
    negative one when greater or equal.  Every product is exact in float64
    (asserted), so each decision is the exact rational one."""
    t = np.asarray(table, dtype=np.float32).astype(np.float64)
    vals = sorted({float(v) for v in t})            # +0 and -0 collapse to one value
    code_of = np.array([min(c for c in range(t.size) if t[c] == v) for v in vals])
    mids = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        m = (lo + hi) / 2.0
        assert Fraction(m) == (Fraction(lo) + Fraction(hi)) / 2, "inexact midpoint"
        assert m != 0.0, "symmetric pair around zero: tie rule undefined"
        assert _sig_bits(m) <= 29, "a * m would not be exact in float64"
        mids.append(m)
    x = np.asarray(x, dtype=np.float64)
    a = np.broadcast_to(np.asarray(a, dtype=np.float64), x.shape).ravel()
    x = x.ravel()
    assert np.all(a >= 0)
    rank = np.zeros(x.size, dtype=np.int64)
    for m in mids:
        thr = a * m
        rank += (x > thr) if m > 0 else (x >= thr)
    return code_of[rank]


def nearest_codes(x, a, table, forms: str = "both") -> np.ndarray:
    """Exact nearest code (R3).  By default both formulations run and must
    agree; ``forms="threshold"`` runs the threshold form alone (the same
    decisions, pinned against the literal form and exact-rational brute force
    by the tests; used for whole tensors at full size, where 16 or 256
    distances per element take too long)."""
    if forms == "threshold":
        return nearest_codes_threshold(x, a, table)
    lit = nearest_codes_literal(x, a, table)
    thr = nearest_codes_threshold(x, a, table)
    bad = np.flatnonzero(lit != thr)
    if bad.size:
        raise AssertionError(f"nearest-code formulations disagree at {bad[:8]}")
    return lit


# --------------------------------------------------------------------------
# packing (R4; nibble order: parity unpinned against external data)
# --------------------------------------------------------------------------
def pack_nibbles(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).ravel()
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, dtype=np.uint8)])
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_nibbles(packed, numel: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).ravel()
    c = np.empty(p.size * 2, dtype=np.uint8)
    c[0::2] = p >> 4
    c[1::2] = p & 15
    return c[:numel]


# --------------------------------------------------------------------------
# quantize_4bit
# --------------------------------------------------------------------------
def quantize_4bit(w, blocksize: int = 64, quant_type: str = "nf4", forms: str = "both"):
    """Returns (packed uint8 [ceil(numel/2)], absmax fp32 [ceil(numel/bs)]).

    "Functional API" (4-bit): per-block absmax, nearest NF4/FP4 code, two codes
    per byte; "What runs natively now": quantize_4bit is one of the ops.
    ``forms`` as for nearest_codes."""
    x = np.asarray(w, dtype=np.float64).ravel()
    table = code_table(quant_type)
    absmax = block_absmax(x, blocksize)
    codes = np.empty(x.size, dtype=np.uint8)
    chunk = _CHUNK if forms == "both" else _CHUNK * 16
    step = max(blocksize, (chunk // blocksize) * blocksize)
    for s in range(0, x.size, step):
        xs = x[s:s + step]
        a = np.repeat(absmax[s // blocksize: s // blocksize + -(-xs.size // blocksize)],
                      blocksize)[: xs.size]
        codes[s:s + step] = nearest_codes(xs, a, table, forms)
    a32 = absmax.astype(np.float32)
    assert np.array_equal(a32.astype(np.float64), absmax)   # absmax is exact in fp32
    return pack_nibbles(codes), a32


# --------------------------------------------------------------------------
# double quantization (R5, R6)
# --------------------------------------------------------------------------
def mean_fixed_tree(absmax) -> np.float32:
    """fp32(S / n), S summed in float64 in the fixed tree of R5."""
    level = [float(v) for v in np.asarray(absmax, dtype=np.float32)]
    n = len(level)
    if n == 0:
        raise ValueError("empty absmax")
    while len(level) > 1:
        nxt = []
        for i in range(0, len(level), MEAN_FANIN):
            s = 0.0
            for v in level[i:i + MEAN_FANIN]:
                s += v
            nxt.append(s)
        level = nxt
    return np.float32(level[0] / n)


def double_quant(absmax, blocksize2: int = 256, code2=None, forms: str = "both"):
    """Returns (q uint8 [n], absmax2 fp32 [ceil(n/bs2)], offset fp32).

    "Functional API" (Double Quantization): double_quant(absmax,
    double_quant_block=256) quantizes the scales; "Features": double
    quantization saves on scales."""
    a = np.asarray(absmax, dtype=np.float32).ravel()
    code2 = linear8_table() if code2 is None else np.asarray(code2, dtype=np.float32)
    offset = mean_fixed_tree(a)
    c = (a - offset).astype(np.float32)                  # fp32 subtraction, RN
    s = block_absmax(c.astype(np.float64), blocksize2)   # exact
    s_el = np.repeat(s, blocksize2)[: a.size]
    q = nearest_codes(c.astype(np.float64), s_el, code2, forms)
    return q.astype(np.uint8), s.astype(np.float32), offset


def dequant_absmax(q, absmax2, offset, code2=None, blocksize2: int = 256) -> np.ndarray:
    """R6: a_hat = fp32(fp32(code2[q] * s_g) + offset).  "Functional API":
    dequant_absmax restores the scales."""
    q = np.asarray(q, dtype=np.int64).ravel()
    code2 = linear8_table() if code2 is None else np.asarray(code2, dtype=np.float32)
    s = np.repeat(np.asarray(absmax2, dtype=np.float32), blocksize2)[: q.size]
    prod = code2[q] * s                                   # fp32 multiply, RN
    return (prod + np.float32(offset)).astype(np.float32) # fp32 add, RN


# --------------------------------------------------------------------------
# 8-bit blockwise codec (R10, R11)
# --------------------------------------------------------------------------
def dynamic_tree_table() -> np.ndarray:
    """R11: the signed dynamic-tree 8-bit table.  After the sign, a run of e
    zero bits (e = 0..6) selects the decimal exponent and the bits after the
    first one bit (6 - e of them) a linear fraction: the centre of bin j of
    [0.1, 1] cut into 2^(6-e) equal bins.  Values 10^-e * centre, their
    negatives, 0 and 1, rounded once to fp32 and sorted (256 values)."""
    mags = []
    for e in range(7):
        bins = 2 ** (6 - e)
        width = 0.9 / bins
        for j in range(bins):
            centre = 0.1 + width * (j + 0.5)
            mags.append(np.float32(centre * 10.0 ** (-e)))
    vals = [np.float32(0.0), np.float32(1.0)] + mags + [np.float32(-m) for m in mags]
    t = np.array(sorted(set(float(v) for v in vals)), dtype=np.float32)
    assert t.size == 256
    return t


def quantize_blockwise(x, blocksize: int, code=None):
    """R10: 8-bit blockwise codec.  "What runs natively now": quantize_blockwise
    (8-bit); "Known failures": the reference is an exact float64 nearest-code
    search.  absmax[b] = max |x| over block b (fp32, exact); q = exact nearest
    code of x / absmax[b] (R3's tie rule; a zero block takes the code of 0).
    Returns (q uint8 [n], absmax fp32 [ceil(n / blocksize)])."""
    x = np.asarray(x, dtype=np.float64).ravel()
    code = linear8_table() if code is None else np.asarray(code, dtype=np.float32)
    a = block_absmax(x, blocksize)
    a_el = np.repeat(a, blocksize)[: x.size]
    q = nearest_codes(x, a_el, code)
    return q.astype(np.uint8), a.astype(np.float32)


def dequantize_blockwise(q, absmax, blocksize: int, code=None, out_dtype: str = "fp32"):
    """R10: w = fp32(code[q] * absmax[block]), then rounded to the output type."""
    q = np.asarray(q, dtype=np.int64).ravel()
    code = linear8_table() if code is None else np.asarray(code, dtype=np.float32)
    a = np.repeat(np.asarray(absmax, dtype=np.float32), blocksize)[: q.size]
    return _cast_out((code[q] * a).astype(np.float32), out_dtype)


# --------------------------------------------------------------------------
# dequantize_4bit (R7)
# --------------------------------------------------------------------------
def dequantize_4bit(packed, absmax_hat, numel: int, blocksize: int,
                    quant_type: str = "nf4", out_dtype: str = "fp32"):
    """w = fp32(T[code] * a_hat), then bf16/fp16 by RNE if asked.  bf16 is
    returned as uint16 bit patterns.  "What runs natively now": dequantize_4bit."""
    table = code_table(quant_type).astype(np.float64)
    codes = unpack_nibbles(packed, numel)
    a = np.repeat(np.asarray(absmax_hat, dtype=np.float32).astype(np.float64),
                  blocksize)[:numel]
    w32 = (table[codes] * a).astype(np.float32)   # exact product, one rounding
    return _cast_out(w32, out_dtype)


def _cast_out(w32, out_dtype):
    if out_dtype == "fp32":
        return w32
    if out_dtype == "bf16":
        return f32_to_bf16_bits(w32)
    if out_dtype == "fp16":
        return f32_to_f16(w32)
    raise ValueError(out_dtype)


def dequantize_rows(packed, absmax_hat, N: int, K: int, blocksize: int,
                    quant_type: str, rows) -> np.ndarray:
    """fp32 dequantized rows ``rows`` of an [N, K] weight (K % blocksize == 0,
    so no block straddles a row)."""
    assert K % blocksize == 0 and K % 2 == 0
    rows = np.asarray(rows, dtype=np.int64)
    p = np.asarray(packed, dtype=np.uint8).reshape(N, K // 2)[rows]
    a = np.asarray(absmax_hat, dtype=np.float32).reshape(N, K // blocksize)[rows]
    return np.stack([dequantize_4bit(p[i], a[i], K, blocksize, quant_type)
                     for i in range(rows.size)]) if rows.size else np.zeros((0, K), np.float32)


# --------------------------------------------------------------------------
# Embedding4bit (R13)
# --------------------------------------------------------------------------
def embedding_4bit(idx, packed, absmax_hat, V: int, D: int, blocksize: int,
                   quant_type: str = "nf4", out_dtype: str = "fp32"):
    """R13: "Quantized Embeddings": out[t] = row idx[t] of the dequantized
    [V, D] table (dequantize_4bit of the flattened table, R7), rounded to the
    output type; an index outside [0, V) gives a row of zeros."""
    idx = np.asarray(idx, dtype=np.int64).ravel()
    W = dequantize_4bit(packed, absmax_hat, V * D, blocksize, quant_type).reshape(V, D)
    out = np.zeros((idx.size, D), dtype=np.float32)
    ok = (idx >= 0) & (idx < V)
    out[ok] = W[idx[ok]]
    return _cast_out(out, out_dtype)


# --------------------------------------------------------------------------
# gemv_4bit / gemm_4bit (R8)
# --------------------------------------------------------------------------
def matmul_4bit(X, packed, absmax_hat, N: int, K: int, blocksize: int,
                quant_type: str = "nf4") -> np.ndarray:
    """Y[M, N] = X[M, K] @ W_hat[N, K]^T in float64.  "What runs natively now":
    gemv_4bit and gemm_4bit replace dequantize-then-linear, which is therefore
    the definition they are checked against."""
    W = dequantize_4bit(packed, absmax_hat, N * K, blocksize, quant_type).reshape(N, K)
    return np.asarray(X, dtype=np.float64).reshape(-1, K) @ W.astype(np.float64).T


def matmul_4bit_backward(dY, packed, absmax_hat, N: int, K: int, blocksize: int,
                         quant_type: str = "nf4") -> np.ndarray:
    """dX[M, K] = dY[M, N] @ W_hat[N, K] in float64.  "What runs natively
    now" (gemm_4bit_backward) and the paragraph after it: the op's default is
    grad_output @ dequantize_4bit(B), which is therefore its definition."""
    W = dequantize_4bit(packed, absmax_hat, N * K, blocksize, quant_type).reshape(N, K)
    return np.asarray(dY, dtype=np.float64).reshape(-1, N) @ W.astype(np.float64)


def matmul_4bit_rows(X, packed, absmax_hat, N: int, K: int, blocksize: int,
                     quant_type: str, rows) -> np.ndarray:
    """Columns ``rows`` of Y (output features), for checks at full size."""
    W = dequantize_rows(packed, absmax_hat, N, K, blocksize, quant_type, rows)
    return np.asarray(X, dtype=np.float64).reshape(-1, K) @ W.astype(np.float64).T
