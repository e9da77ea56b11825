"""GPU parity of the general 8-bit blockwise codec (quantize_blockwise /
dequantize_blockwise) against the CPU oracle: bit-exact codes, block absmax
and dequantized values, through the C ABI on the caller's stream."""
import numpy as np
import pytest
import torch

import oracle as O
from quantized_matvec_amd import qmv

pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def bits32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def table(name):
    """(list for the binding, fp32 array for the oracle).  The binding's
    None means its default table, (k - 127) / 127."""
    if name == "linear":
        return None, O.linear8_table()
    if name == "dynamic":
        return qmv.dynamic_tree_code(), O.dynamic_tree_table()
    # a random codebook on a 2^-12 grid with 0 and +-1 in it: every midpoint
    # is exact in few bits, and adjacent values are unevenly spaced
    rng = np.random.default_rng(77)
    pool = np.concatenate([np.arange(-4095, 0), np.arange(1, 4096)])
    k = np.sort(np.concatenate([rng.choice(pool, 253, replace=False), [-4096, 0, 4096]]))
    t = (k / 4096.0).astype(np.float32)
    return t.tolist(), t


def mixed_data(n, dtype, seed, bs):
    """Gaussian values with per-block scales spanning many binades, an exact
    zero block, exact zeros inside a live block and a tiny-valued block."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(n)
    nb = -(-n // bs)
    v *= np.repeat(10.0 ** rng.uniform(-5, 3, size=nb), bs)[:n]
    if nb >= 4:
        v[bs:2 * bs] = 0.0
        v[2 * bs + 3:2 * bs + 9] = 0.0
        v[3 * bs:4 * bs] *= 1e-33 if dtype == "fp32" else 1.0
    t = torch.from_numpy(v).to(torch.float32)
    if dtype != "fp32":
        t = t.clamp(-6e4, 6e4).to(TDT[dtype])
    return t


def check_quantize(A_cpu, bs, tname):
    code_list, code = table(tname)
    q, absmax = qmv.quantize_blockwise(A_cpu.cuda(), bs, code_list)
    torch.cuda.synchronize()
    q_ref, a_ref = O.quantize_blockwise(f64(A_cpu), bs, code)
    assert np.array_equal(bits32(absmax.cpu().numpy()), bits32(a_ref))
    got = q.cpu().numpy()
    bad = np.flatnonzero(got != q_ref)
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[:5]}"
    return q, absmax, q_ref, a_ref


@pytest.mark.parametrize("tname", ["linear", "dynamic", "random"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("bs", [32, 64, 256, 2048, 4096])
def test_quantize_blockwise_bitexact(tname, dtype, bs):
    check_quantize(mixed_data(5 * 4096 + 40, dtype, seed=bs + len(tname), bs=bs), bs, tname)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 255, 4097, 65536 + 5])
@pytest.mark.parametrize("tname", ["linear", "dynamic"])
def test_quantize_blockwise_ragged(n, tname):
    check_quantize(mixed_data(n, "bf16", seed=n, bs=64), 64, tname)


@pytest.mark.parametrize("tname", ["linear", "dynamic"])
def test_quantize_blockwise_exact_on_a_million_values(tname):
    """The exactness workload of the blockwise codec: 1,048,576 fp32 normal
    values at the default blocksize 4096, every code exact."""
    A = torch.from_numpy(np.random.default_rng(2024).standard_normal(1 << 20)).to(torch.float32)
    check_quantize(A, 4096, tname)


def test_quantize_blockwise_ties_and_extremes():
    """Exact midpoints of adjacent dynamic-tree values (times a power of two)
    go to the smaller magnitude; +-absmax take the extreme codes."""
    code_list, code = table("dynamic")
    mids = (code[:-1].astype(np.float64) + code[1:].astype(np.float64)) / 2.0
    mids = mids[mids.astype(np.float32).astype(np.float64) == mids]   # ties fp32 can hold
    assert mids.size > 100
    v = np.concatenate([[8.0, -8.0], mids * 8.0, [0.0, -0.0]])
    v = np.concatenate([v, np.zeros(512 - v.size)])
    check_quantize(torch.from_numpy(v).to(torch.float32), 512, "dynamic")


@pytest.mark.parametrize("tname", ["linear", "dynamic", "random"])
@pytest.mark.parametrize("out", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("n,bs", [(64 * 300 + 7, 64), (4096 * 3 + 16, 4096), (33, 32), (16, 32)])
def test_dequantize_blockwise_bitexact(tname, out, n, bs):
    code_list, code = table(tname)
    rng = np.random.default_rng(n + bs)
    q = rng.integers(0, 256, n).astype(np.uint8)
    nb = -(-n // bs)
    absmax = (np.abs(rng.standard_normal(nb)) * 10.0 ** rng.uniform(-4, 2, nb)).astype(np.float32)
    absmax[0] = 0.0
    got = qmv.dequantize_blockwise(torch.from_numpy(q).cuda(), torch.from_numpy(absmax).cuda(), bs,
                                   code_list, TDT[out])
    torch.cuda.synchronize()
    want = O.dequantize_blockwise(q, absmax, bs, code, out)
    g = got.cpu()
    if out == "fp32":
        assert np.array_equal(bits32(g.numpy()), bits32(want))
    else:
        gb = g.view(torch.int16).numpy().view(np.uint16)
        wb = np.asarray(want).view(np.uint16) if out == "fp16" else np.asarray(want, dtype=np.uint16)
        assert np.array_equal(gb, wb)


@pytest.mark.parametrize("tname", ["linear", "dynamic"])
def test_roundtrip_on_device(tname):
    """quantize then dequantize on the GPU, compared with the oracle's pair."""
    code_list, code = table(tname)
    A = mixed_data(64 * 513 + 11, "bf16", seed=9, bs=256)
    q, absmax, q_ref, a_ref = check_quantize(A, 256, tname)
    w = qmv.dequantize_blockwise(q, absmax, 256, code_list, torch.bfloat16)
    torch.cuda.synchronize()
    want = O.dequantize_blockwise(q_ref, a_ref, 256, code, "bf16")
    assert np.array_equal(w.cpu().view(torch.int16).numpy().view(np.uint16), np.asarray(want, dtype=np.uint16))


def test_quantize_blockwise_large_sampled():
    """Past the launch's grid cap (65536 tiles of 2048 elements), so the
    grid-stride loop runs: every sampled block's absmax and codes exact, and
    a dequantize of the same blocks exact."""
    n = (1 << 27) + (1 << 20) + 3
    bs = 1024
    g = torch.Generator().manual_seed(3)
    A_cpu = torch.randn(n, generator=g, dtype=torch.float32).to(torch.bfloat16)
    code_list, code = table("dynamic")
    q, absmax = qmv.quantize_blockwise(A_cpu.cuda(), bs, code_list)
    w = qmv.dequantize_blockwise(q, absmax, bs, code_list, torch.float32)
    torch.cuda.synchronize()
    nb = -(-n // bs)
    blocks = np.unique(np.concatenate([[0, nb // 2, nb - 2, nb - 1],
                                       np.random.default_rng(4).integers(0, nb, 60)]))
    qc, ac, wc = q.cpu().numpy(), absmax.cpu().numpy(), w.cpu().numpy()
    for b in blocks:
        lo, hi = int(b) * bs, min(n, (int(b) + 1) * bs)
        q_ref, a_ref = O.quantize_blockwise(f64(A_cpu[lo:hi]), bs, code)
        assert bits32(ac[b:b + 1]).tolist() == bits32(a_ref).tolist(), b
        assert np.array_equal(qc[lo:hi], q_ref), b
        assert np.array_equal(bits32(wc[lo:hi]), bits32(O.dequantize_blockwise(q_ref, a_ref, bs, code))), b
