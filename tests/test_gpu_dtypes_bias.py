"""GPU parity of the fp16 / fp32 compute paths of gemv_4bit / gemm_4bit /
gemm_4bit_backward and of the bias epilogue, through the C ABI.

Tolerances (relative L2 against the float64 oracle): fp16 activations with
fp32 outputs 2e-3 (the weights are rounded to fp16, 2^-11 relative, the
activations are exact, accumulation is fp32); fp32 activations 1e-5 (fp32
weights, products and sums); 16-bit outputs 2e-2 as elsewhere.  Exact pins:
identity rows of fp16 A return the fp16-rounded dequantized weight (tile and
split-K kernels) or fp32(a_hat * fp16(T)) (narrow kernel) bit for bit, and a
bias changes the output exactly by one fp32 addition before the one rounding
to the output type."""
import numpy as np
import pytest
import torch

import oracle as O
from bounds import check_backward, check_matmul
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def oracle_state(W64, bs, qt, dq, bs2=256):
    packed, absmax = O.quantize_4bit(W64, bs, qt)
    if dq:
        q, a2, off = O.double_quant(absmax, bs2)
        return packed, O.dequant_absmax(q, a2, off, None, bs2)
    return packed, absmax


def upload_state(packed, absmax, shape, dtype, bs, qt):
    st = qmv.QuantState(tuple(shape), dtype, bs, qt, absmax=torch.from_numpy(absmax).cuda())
    return torch.from_numpy(packed).cuda(), st


def f16_bits(a32):
    return np.asarray(a32, dtype=np.float32).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- fp16 activations
@pytest.mark.parametrize("M", [1, 4, 8, 16, 17, 33, 64, 65, 300])
@pytest.mark.parametrize("dq", [False, True])
def test_gemm_fp16_parity(M, dq):
    """Every gemm kernel with fp16 A: narrow (M <= 16), split-K (<= 64),
    tile (the rest); N = 200 ends on a partial 32-column group."""
    N, K, bs = 200, 512, 64
    W = synth.gaussian((N, K), 0.02, 300 + M, "fp16")
    A = synth.gaussian((M, K), 1.0, 301 + M, "fp16")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=dq)
    Wh = O.dequantize_4bit(p_ref, ahat, N * K, bs, "nf4").reshape(N, K)
    C = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=torch.float32)
    check_matmul(f64(C), f64(A), Wh, "fp16", "fp32", f"M={M} dq={dq}")
    Ch = qmv.gemm_4bit(A.cuda(), packed, st)
    assert Ch.dtype == torch.float16
    check_matmul(f64(Ch), f64(A), Wh, "fp16", "fp16", f"M={M} dq={dq} fp16 out")


@pytest.mark.parametrize("rows", [17, 64, 200])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_gemm_fp16_identity_rows_exact(qt, rows):
    """Split-K and tile kernels multiply the fp16 dequantize_4bit weights."""
    N, K = 300, 256
    W = synth.gaussian((N, K), 0.02, 309, "bf16")
    p_ref, a_ref = O.quantize_4bit(f64(W), 64, qt)
    packed, st = upload_state(p_ref, a_ref, (N, K), torch.float16, 64, qt)
    A = torch.eye(K, dtype=torch.float16)[:rows]
    C = qmv.gemm_4bit(A.cuda(), packed, st).cpu().view(torch.int16).numpy().view(np.uint16)
    What = np.asarray(O.dequantize_4bit(p_ref, a_ref, N * K, 64, qt, "fp16")).view(np.uint16).reshape(N, K)
    assert np.array_equal(C, What[:, :rows].T)


@pytest.mark.parametrize("rows", [1, 8, 16])
def test_gemm_fp16_narrow_identity_rows_exact(rows):
    """The narrow kernel: fp32(a_hat * fp16(T[code])) per identity row."""
    N, K, bs = 300, 256, 64
    W = synth.gaussian((N, K), 0.02, 319, "bf16")
    p_ref, a_ref = O.quantize_4bit(f64(W), bs, "nf4")
    packed, st = upload_state(p_ref, a_ref, (N, K), torch.float16, bs, "nf4")
    A = torch.eye(K, dtype=torch.float16)[5:5 + rows]
    t16 = O.code_table("nf4").astype(np.float32).astype(np.float16).astype(np.float32)
    codes = O.unpack_nibbles(p_ref, N * K).reshape(N, K)
    scale = np.repeat(a_ref.astype(np.float32).reshape(N, K // bs), bs, axis=1)
    w = t16[codes] * scale + np.float32(0)
    want = np.ascontiguousarray(w[:, 5:5 + rows].T)
    C = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(C.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("M", [4, 8])
def test_gemv_fp16_takes_the_narrow_kernel(M):
    """fp16 x with 4..8 rows runs on the matrix cores like bf16: the result
    equals gemm_4bit's for the same rows bit for bit."""
    N, K = 512, 1024
    W = synth.gaussian((N, K), 0.02, 330, "fp16")
    x = synth.gaussian((M, K), 1.0, 331, "fp16").cuda()
    packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4", double_quant=True)
    y = qmv.gemv_4bit(x, packed, st, out_dtype=torch.float32)
    C = qmv.gemm_4bit(x, packed, st, out_dtype=torch.float32)
    assert torch.equal(y, C)


@pytest.mark.parametrize("M", [1, 100, 300])
def test_backward_fp16(M):
    N, K, bs = 256, 384, 64
    W = synth.gaussian((N, K), 0.02, 340 + M, "fp16")
    dY = synth.gaussian((M, N), 1.0, 341 + M, "fp16")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", True)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=True)
    Wh = O.dequantize_4bit(p_ref, ahat, N * K, bs, "nf4").reshape(N, K)
    dX = qmv.gemm_4bit_backward(dY.cuda(), packed, st, out_dtype=torch.float32)
    check_backward(f64(dX), f64(dY), Wh, "fp16", "fp32", f"M={M}")
    # identity rows of dY return rows of the fp16 dequantized weight exactly
    I = torch.eye(N, dtype=torch.float16)[:M if M <= N else N].cuda()
    rows = I.shape[0]
    dXi = qmv.gemm_4bit_backward(I, packed, st).cpu().view(torch.int16).numpy().view(np.uint16)
    What = np.asarray(O.dequantize_4bit(p_ref, ahat, N * K, bs, "nf4", "fp16")).view(np.uint16).reshape(N, K)
    assert np.array_equal(dXi, What[:rows])


# ---------------------------------------------------------------- fp32 activations
@pytest.mark.parametrize("M", [1, 8, 9, 20, 129, 300])
@pytest.mark.parametrize("od", ["fp32", "bf16"])
def test_gemm_fp32_parity(M, od):
    """fp32 A: fp32 weights, products and sums (up to 8 rows on the fp32 gemv
    kernel, more on the fp32 matrix cores in 128 x 128 tiles: 129 and 300
    end on partial row tiles, N = 200 on a partial column tile)."""
    N, K, bs = 200, 512, 64
    W = synth.gaussian((N, K), 0.02, 350 + M, "fp32")
    A = synth.gaussian((M, K), 1.0, 351 + M, "fp32")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", True)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=True)
    ref = O.matmul_4bit(f64(A), p_ref, ahat, N, K, bs, "nf4")
    C = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=TDT[od])
    assert C.shape == (M, N)
    check_matmul(f64(C), f64(A), O.dequantize_4bit(p_ref, ahat, N * K, bs, "nf4").reshape(N, K),
                 "fp32", od, f"M={M}")
    if od == "fp32":      # fp32 products and sums: far inside the bound
        assert rel_l2(f64(C), ref) <= 1e-5


# ---------------------------------------------------------------- bias epilogue
CASES = [  # (entry, x dtype, M): the kernel each one reaches
    ("gemv", "bf16", 1),    # M = 1 kernel
    ("gemv", "fp16", 1),
    ("gemv", "bf16", 2),    # table kernel
    ("gemv", "fp16", 3),
    ("gemv", "bf16", 6),    # narrow MFMA kernel
    ("gemv", "fp32", 3),    # fp32 kernel
    ("gemm", "bf16", 12),   # narrow
    ("gemm", "fp16", 40),   # split-K
    ("gemm", "bf16", 130),  # tile
    ("gemm", "fp32", 11),   # fp32 matrix cores
]


@pytest.mark.parametrize("entry,xd,M", CASES)
@pytest.mark.parametrize("od", ["fp32", "bf16", "fp16"])
def test_bias_is_one_add_before_the_rounding(entry, xd, M, od):
    N, K, bs = 160, 512, 64
    W = synth.gaussian((N, K), 0.02, 360 + M, "bf16")
    x = synth.gaussian((M, K), 1.0, 361 + M, xd).cuda()
    bias = synth.gaussian((N,), 0.5, 362 + M, od).cuda()
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=True)
    f = qmv.gemv_4bit if entry == "gemv" else qmv.gemm_4bit
    acc = f(x, packed, st, out_dtype=torch.float32)             # the fp32 result
    got = f(x, packed, st, out_dtype=TDT[od], bias=bias)
    want = (acc + bias.float()).to(TDT[od])                    # one fp32 add, one rounding
    assert torch.equal(got.view(-1).cpu(), want.view(-1).cpu()), (entry, xd, M, od)
    # and against the oracle
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", True)
    Wh = O.dequantize_4bit(p_ref, ahat, N * K, bs, "nf4").reshape(N, K)
    check_matmul(f64(got), f64(x), Wh, xd, od, f"{entry} {xd} M={M} {od}", bias=f64(bias))


def test_bias_wrong_shape_is_refused():
    N, K = 64, 128
    W = synth.gaussian((N, K), 0.02, 370, "bf16")
    packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4")
    x = synth.gaussian((1, K), 1.0, 371, "bf16").cuda()
    with pytest.raises(ValueError):
        qmv.gemv_4bit(x, packed, st, bias=torch.zeros(N + 1, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        qmv.gemv_4bit(x, packed, st, bias=torch.zeros(N, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("rows", [9, 128, 200])
@pytest.mark.parametrize("dq", [False, True])
def test_gemm_fp32_identity_rows_exact(rows, dq):
    """Identity rows of fp32 A return the fp32 dequantized weight rows bit for
    bit: each output is 1 * w plus exact zeros."""
    N, K, bs = 300, 256, 64
    W = synth.gaussian((N, K), 0.02, 380 + rows, "fp32")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=dq)
    A = torch.eye(K, dtype=torch.float32)[:rows].cuda()
    C = qmv.gemm_4bit(A, packed, st, out_dtype=torch.float32).cpu().numpy()
    What = O.dequantize_4bit(p_ref, ahat, N * K, bs, "nf4").reshape(N, K)
    want = np.ascontiguousarray(What[:, :rows].T) + np.float32(0)   # -0 reads as +0
    assert np.array_equal(C.view(np.uint32), want.view(np.uint32))
