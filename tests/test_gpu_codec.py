"""GPU parity of the codec (quantize_4bit, double quantization, scale
reconstruction, dequantize_4bit) against the CPU oracle: bit-exact, through
the C ABI on the caller's stream."""
import numpy as np
import pytest
import torch

import crafted_inputs
import oracle as O
from quantized_matvec_amd import qmv

pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def bits32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def mixed_data(numel, dtype, seed):
    """Gaussian values with per-block scales spanning many binades, exact zero
    blocks and tiny (subnormal-range) blocks."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(numel)
    scale = 10.0 ** rng.uniform(-6, 3, size=-(-numel // 32))
    v *= np.repeat(scale, 32)[:numel]
    if numel >= 256:
        v[64:128] = 0.0
        v[128:160] *= 1e-35 if dtype == "fp32" else 1.0
    t = torch.from_numpy(v).to(torch.float32)
    if dtype != "fp32":
        t = t.clamp(-6e4, 6e4).to(TDT[dtype])
    return t


def check_quantize(W_cpu, bs, qt):
    W = W_cpu.cuda()
    packed, st = qmv.quantize_4bit(W, bs, qt)
    torch.cuda.synchronize()
    p_ref, a_ref = O.quantize_4bit(f64(W_cpu), bs, qt)
    assert np.array_equal(bits32(st.absmax.cpu().numpy()), bits32(a_ref))
    got = packed.cpu().numpy()
    bad = np.flatnonzero(got != p_ref)
    assert bad.size == 0, f"{bad.size} packed bytes differ, first at {bad[:5]}"
    return packed, st, p_ref, a_ref


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("bs", [32, 64, 128, 512, 2048, 4096])
def test_quantize_bitexact_blocksizes(dtype, qt, bs):
    check_quantize(mixed_data(3 * 4096 + 96, dtype, seed=bs), bs, qt)


@pytest.mark.parametrize("numel", [1, 2, 7, 33, 64, 65, 1023, 4097, 65536 + 17])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_ragged_sizes(numel, qt):
    check_quantize(mixed_data(numel, "bf16", seed=numel), 64, qt)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_constructed_ties_fp32(qt):
    """x = absmax * midpoint exactly (fp32): the tie goes toward zero."""
    table = O.code_table(qt)
    vals = sorted({float(v) for v in table})
    rows = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        m = (lo + hi) / 2
        for a in (1.0, 2.0 ** -9, 2.0 ** 11, 2.0 ** -126):
            x = m * a
            if float(np.float32(x)) == x:
                blk = np.zeros(64)
                blk[0] = a
                blk[1:] = x
                rows.append(blk)
    W = torch.from_numpy(np.concatenate(rows)).to(torch.float32)
    assert len(rows) > 4
    check_quantize(W, 64, qt)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_exhaustive_bf16_pairs(qt):
    """Every bf16 |x| <= a, both signs, for all 128 bf16 absmax mantissas in
    [1, 2) and a few other binades: each block holds a at slot 0 and 63 test
    values.  The decision depends only on (x, a)."""
    blocks = []
    for scale_bits in (0x3F80, 0x0080, 0x7E80):         # binade of 1, 2^-126, 2^126
        for mant in range(128) if scale_bits == 0x3F80 else (0, 77, 127):
            abits = scale_bits | mant
            x = np.arange(0, abits + 1, dtype=np.uint32).astype(np.uint16)
            x = np.concatenate([x, x | 0x8000])
            pad = (-x.size) % 63
            x = np.concatenate([x, np.zeros(pad, np.uint16)]).reshape(-1, 63)
            blk = np.empty((x.shape[0], 64), np.uint16)
            blk[:, 0] = abits
            blk[:, 1:] = x
            blocks.append(blk.ravel())
    bits = np.concatenate(blocks)
    W = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    check_quantize(W, 64, qt)


# ---------------------------------------------------------------- double quant
def dq_case(n, bs2, seed, code2=None):
    rng = np.random.default_rng(seed)
    a = (np.abs(rng.standard_normal(n)) * 0.02).astype(np.float32)
    if n > 600:
        a[300:600] = a[300]            # a run of equal scales (zero group parts)
    ag = torch.from_numpy(a).cuda()
    q, a2, off, c2 = qmv.double_quant(ag, bs2, code2)
    torch.cuda.synchronize()
    q_ref, a2_ref, off_ref = O.double_quant(a, bs2, code2)
    assert bits32(off.cpu().numpy())[0] == bits32([off_ref])[0]
    assert np.array_equal(bits32(a2.cpu().numpy()), bits32(a2_ref))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    table = O.linear8_table() if code2 is None else np.asarray(code2, np.float32)
    assert np.array_equal(bits32(c2.cpu().numpy()), bits32(table))
    return q, a2, off, c2


@pytest.mark.parametrize("n", [1, 2, 255, 256, 257, 4096, 65537, 70001, 256 * 4096,
                               256 * 4096 + 1])
def test_double_quant_bitexact_sizes(n):
    """Up to 4096 first-level runs the encode launch combines the runs; the
    last size takes the separate top-level launch."""
    dq_case(n, 256, seed=n)


@pytest.mark.parametrize("n", [5000, 70001])
def test_double_quant_mean_wide_exponents(n):
    """Scales whose exponents span too far for an exact float64 sum: the
    partial sums round, so only the fixed tree order gives the oracle's mean
    (both the first-level runs and the levels above take the ordered path)."""
    rng = np.random.default_rng(n)
    a = (np.abs(rng.standard_normal(n)) * 0.02).astype(np.float32)
    a[::97] = np.float32(3e-30)
    a[5] = np.float32(7e9)
    ag = torch.from_numpy(a).cuda()
    q, a2, off, c2 = qmv.double_quant(ag, 256)
    torch.cuda.synchronize()
    q_ref, a2_ref, off_ref = O.double_quant(a, 256)
    assert bits32(off.cpu().numpy())[0] == bits32([off_ref])[0]
    assert np.array_equal(bits32(a2.cpu().numpy()), bits32(a2_ref))
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("which", ["two_level", "three_level"])
def test_double_quant_mean_crafted_order(which):
    """Scales built so that every other summation order (flat, pairwise,
    other fan-ins, a pairwise upper level) rounds the fp32 mean differently
    from the fixed 256-run tree (the oracle pins assert each difference):
    the offset must be the tree's, 16384.0 and 64.0."""
    a = getattr(crafted_inputs, "mean_" + which)()
    q, a2, off, c2 = qmv.double_quant(torch.from_numpy(a).cuda(), 256)
    torch.cuda.synchronize()
    q_ref, a2_ref, off_ref = O.double_quant(a, 256, forms="threshold")
    assert float(off_ref) == (16384.0 if which == "two_level" else 64.0)
    assert bits32(off.cpu().numpy())[0] == bits32([off_ref])[0]
    assert np.array_equal(bits32(a2.cpu().numpy()), bits32(a2_ref))
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("bs2", [32, 64, 512, 4096])
def test_double_quant_group_sizes(bs2):
    dq_case(20000, bs2, seed=bs2)


def test_double_quant_custom_table():
    code2 = ((np.arange(256) - 128) / 128.0).astype(np.float32).tolist()
    dq_case(5000, 256, seed=3, code2=code2)


def test_double_quant_constant_scales_zero_groups():
    a = np.full(1000, 0.25, np.float32)
    q, a2, off, _ = qmv.double_quant(torch.from_numpy(a).cuda(), 256)
    assert float(off.item()) == 0.25
    assert torch.all(a2 == 0).item() and torch.all(q == 127).item()


# ---------------------------------------------------------------- dequantize
def assert_same_bits(got, ref, what):
    got = np.asarray(got).ravel()
    ref = np.asarray(ref).ravel()
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (f"{what}: {bad.size} of {ref.size} differ; first indices {bad[:6]}, "
                           f"got {got[bad[:6]]}, want {ref[bad[:6]]}")


@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("out", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("numel", [64 * 1024, 64 * 1000 + 37])
def test_dequantize_bitexact(dq, qt, out, numel):
    Wc = mixed_data(numel, "bf16", seed=numel + dq)
    packed, st = qmv.quantize_4bit(Wc.cuda(), 64, qt, double_quant=dq)
    w = qmv.dequantize_4bit(packed, st, out_dtype=TDT[out])
    ahat_gpu = qmv.dequantize_absmax(st)
    torch.cuda.synchronize()
    p_ref, a_ref = O.quantize_4bit(f64(Wc), 64, qt)
    if dq:
        q, a2, off = O.double_quant(a_ref, 256)
        ahat = O.dequant_absmax(q, a2, off, None, 256)
    else:
        ahat = a_ref
    assert_same_bits(bits32(ahat_gpu.cpu().numpy()), bits32(ahat), "scales")
    ref = O.dequantize_4bit(p_ref, ahat, numel, 64, qt, out)
    if out == "fp32":
        assert_same_bits(bits32(w.cpu().numpy()), bits32(ref), "fp32 weights")
    else:
        got = w.cpu().view(torch.int16).numpy().view(np.uint16)
        assert_same_bits(got, np.asarray(ref).view(np.uint16), out + " weights")


def test_quantize_dequantize_roundtrip_invariants():
    """The absmax element of each block comes back as +-absmax exactly and
    zeros stay zero."""
    Wc = mixed_data(64 * 512, "bf16", seed=99)
    packed, st = qmv.quantize_4bit(Wc.cuda(), 64, "nf4")
    w = qmv.dequantize_4bit(packed, st, out_dtype=torch.float32).cpu().numpy().reshape(-1, 64)
    x = f64(Wc).reshape(-1, 64)
    idx = np.abs(x).argmax(axis=1)
    rows = np.arange(x.shape[0])
    assert np.array_equal(w[rows, idx].astype(np.float64), x[rows, idx])
    assert np.all(w[x == 0] == 0)
