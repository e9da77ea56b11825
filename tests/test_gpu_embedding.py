"""GPU parity of embedding_4bit (rows of a 4-bit quantized embedding table)
against the CPU oracle: bit for bit, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def bits(t):
    t = t.cpu()
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def want_bits(a, od):
    a = np.asarray(a)
    if od == "fp32":
        return a.astype(np.float32).view(np.uint32)
    if od == "fp16":
        return a.view(np.uint16)
    return a.astype(np.uint16)


def check(V, D, bs, qt, dq, od, idx, seed):
    W = synth.gaussian((V, D), 1.0, seed, "bf16")
    packed, st = qmv.quantize_4bit(W.cuda(), bs, qt, double_quant=dq, blocksize2=256)
    p_ref, a_ref = O.quantize_4bit(f64(W), bs, qt)
    if dq:
        q, a2, off = O.double_quant(a_ref, 256)
        a_ref = O.dequant_absmax(q, a2, off, None, 256)
    idx_t = torch.as_tensor(idx, dtype=torch.int64)
    out = qmv.embedding_4bit(idx_t.cuda(), packed, st, out_dtype=TDT[od])
    torch.cuda.synchronize()
    assert out.shape == tuple(idx_t.shape) + (D,)
    want = O.embedding_4bit(idx_t.numpy(), p_ref, a_ref, V, D, bs, qt, od)
    got = bits(out).reshape(-1, D)
    assert np.array_equal(got, want_bits(want, od).reshape(-1, D))


@pytest.mark.parametrize("od", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("dq", [False, True])
def test_embedding_bitexact(od, qt, dq):
    V, D = 1000, 4096 + 64   # two 2048-element segments and a short third
    rng = np.random.default_rng(1)
    idx = rng.integers(0, V, 300)
    idx[:4] = [0, V - 1, 7, 7]
    check(V, D, 64, qt, dq, od, idx, seed=11)


@pytest.mark.parametrize("D,bs", [(64, 64), (200, 32), (4096, 4096), (45, 32), (1, 32), (3000, 128)])
def test_embedding_widths(D, bs):
    """D a multiple of 8 takes the vector path; 45 and 1 the per-element one
    (rows start mid-byte, blocks straddle rows)."""
    V = 97
    idx = np.random.default_rng(D).integers(0, V, 50)
    check(V, D, bs, "nf4", True, "bf16", idx, seed=20 + D)


def test_embedding_out_of_range_rows_are_zero():
    idx = np.array([[3, -1, 96], [97, 1 << 40, 0]])   # 2-D indices
    check(97, 256, 64, "nf4", False, "fp32", idx, seed=31)


def test_embedding_many_tokens():
    """More output rows than one grid dimension holds (65535): the row loop."""
    V, D = 512, 64
    idx = np.random.default_rng(5).integers(0, V, 70000)
    check(V, D, 64, "fp4", True, "bf16", idx, seed=41)
