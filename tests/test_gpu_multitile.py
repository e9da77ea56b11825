"""Mid-size parity, compared in full, at sizes where every workgroup of the
codec kernels walks several tiles: quantize_4bit and quantize_blockwise run
a grid of at most 8 workgroups per compute unit over tiles of 4096 elements,
dequantize_4bit and dequantize_blockwise at most 8 workgroups (32 waves) per
compute unit over 2048-element chunks per wave.  With 2^26 elements and 256
compute units that is at least 32 tiles per quantize workgroup and 4 chunks
per dequantize wave, so the grid-stride loops, the prefetch of the next tile
and the double-buffered threshold stages all run, and a tile-stride or
buffer-reuse error shows up as a mismatch somewhere in the output.

The input is 64 copies of one 2^20-element pattern, copy i scaled by
2^(i - 32) (exact in bf16): every block of a copy has its own absmax, so a
workgroup that reads or writes the wrong tile gets the wrong scale.  For the
4-bit codec the oracle quantizes the whole tensor.  The 8-bit codec's exact
search over 255 thresholds per element is too slow for 2^26 elements, so
its oracle runs on the pattern: the nearest code of x / a does not change
when x and a are scaled by the same power of two (the quotient is the same
number), so every copy's codes are the pattern's codes; this invariance is
checked on one scaled copy against the oracle as well.  Block maxima and
dequantized outputs are computed by the oracle over the whole tensor."""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from quantized_matvec_amd import qmv

pytestmark = pytest.mark.gpu
P = 1 << 20          # pattern length
COPIES = 64


def bits32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def u16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def assert_equal(got, want, what):
    got = np.asarray(got).ravel()
    want = np.asarray(want).ravel()
    assert got.shape == want.shape, what
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} of {want.size} differ, first at {bad[:6]}"


@functools.lru_cache(maxsize=1)
def tensor():
    """bf16 [64 * 2^20]: copies of a Gaussian pattern with per-256 scales over
    four decades, a zero run and one tiny run, copy i scaled by 2^(i - 32)."""
    rng = np.random.default_rng(2601)
    v = rng.standard_normal(P) * np.repeat(10.0 ** rng.uniform(-2, 2, P // 256), 256)
    v[4096:8192] = 0.0
    v[8192:8192 + 512] *= 1e-20          # tiny, but normal after every scaling
    pat = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16)
    scales = torch.tensor([2.0 ** (i - 32) for i in range(COPIES)], dtype=torch.float32)
    full = (pat.to(torch.float32)[None, :] * scales[:, None]).to(torch.bfloat16).reshape(-1)
    # the scaling is exact: every copy holds the pattern's values times 2^(i - 32)
    assert torch.equal(full[5 * P:6 * P].to(torch.float32), pat.to(torch.float32) * 2.0 ** -27)
    return pat, full


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("dq", [False, True])
def test_quantize_dequantize_4bit_many_tiles(qt, dq):
    _, W = tensor()
    n = W.numel()
    print(f"[multitile] 4-bit {qt} dq={dq} on {n} elements", flush=True)
    packed, st = qmv.quantize_4bit(W.cuda(), 64, qt, double_quant=dq)
    w = qmv.dequantize_4bit(packed, st, out_dtype=torch.bfloat16)
    w32 = qmv.dequantize_4bit(packed, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    p_ref, a_ref = O.quantize_4bit(W.to(torch.float64).numpy(), 64, qt, forms="threshold")
    assert_equal(packed.cpu().numpy(), p_ref, "packed codes")
    if dq:
        q, a2, off = O.double_quant(a_ref, 256, forms="threshold")
        assert_equal(st.absmax_q.cpu().numpy(), q, "scale codes")
        assert_equal(bits32(st.absmax2.cpu().numpy()), bits32(a2), "group scales")
        assert bits32(st.offset.cpu().numpy())[0] == bits32([off])[0]
        ahat = O.dequant_absmax(q, a2, off)
    else:
        assert_equal(bits32(st.absmax.cpu().numpy()), bits32(a_ref), "block absmax")
        ahat = a_ref
    w_ref = O.dequantize_4bit(p_ref, ahat, n, 64, qt)
    assert_equal(bits32(w32.cpu().numpy()), bits32(w_ref), "fp32 weights")
    assert_equal(u16(w), O.f32_to_bf16_bits(w_ref), "bf16 weights")


@pytest.mark.parametrize("table", ["linear", "dynamic"])
@pytest.mark.parametrize("bs", [64, 4096])
def test_blockwise_8bit_many_tiles(table, bs):
    pat, A = tensor()
    code = None if table == "linear" else qmv.dynamic_tree_code()
    print(f"[multitile] 8-bit {table} bs={bs} on {A.numel()} elements", flush=True)
    q, absmax = qmv.quantize_blockwise(A.cuda(), bs, code)
    out = qmv.dequantize_blockwise(q, absmax, bs, code, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    q_pat, _ = O.quantize_blockwise(pat.to(torch.float64).numpy(), bs, code)
    # scale invariance of the exact nearest code, checked on one copy
    q_copy, _ = O.quantize_blockwise(A[7 * P:8 * P].to(torch.float64).numpy(), bs, code)
    assert np.array_equal(q_copy, q_pat)
    a_ref = O.block_absmax(A.to(torch.float64).numpy(), bs).astype(np.float32)
    assert_equal(bits32(absmax.cpu().numpy()), bits32(a_ref), "block maxima")
    assert_equal(q.cpu().numpy(), np.tile(q_pat, COPIES), "8-bit codes")
    want = O.dequantize_blockwise(np.tile(q_pat, COPIES), a_ref, bs, code, "bf16")
    assert_equal(u16(out), want, "bf16 output")
