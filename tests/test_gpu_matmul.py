"""GPU parity of gemv_4bit and gemm_4bit against the CPU oracle (dequantize,
then a float64 matmul), through the C ABI.

Every comparison checks the relative L2 error over the whole output and the
per-element worst-case bound of ``bounds.check_matmul`` (derived from the
weight rounding to the activations' type, fp32 accumulation and the output
rounding).  Exact pins: a one-hot x returns a column of the dequantized
weight bit for bit (fp32 path), and identity rows of A return rows of the
bf16-rounded dequantized weight bit for bit (gemm)."""
import numpy as np
import pytest
import torch

import oracle as O
from bounds import check_matmul, rel_l2
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def oracle_state(W64, bs, qt, dq, bs2=256):
    """Oracle quantization of the whole weight: (packed, a_hat)."""
    packed, absmax = O.quantize_4bit(W64, bs, qt)
    if dq:
        q, a2, off = O.double_quant(absmax, bs2)
        return packed, O.dequant_absmax(q, a2, off, None, bs2)
    return packed, absmax


def w_hat(packed, ahat, N, K, bs, qt):
    """The oracle's fp32 dequantized weight [N, K] as float64."""
    return O.dequantize_4bit(packed, ahat, N * K, bs, qt).reshape(N, K).astype(np.float64)


def upload_state(packed, absmax, shape, dtype, bs, qt):
    st = qmv.QuantState(tuple(shape), dtype, bs, qt, absmax=torch.from_numpy(absmax).cuda())
    return torch.from_numpy(packed).cuda(), st


def gaussian(shape, sigma, seed, dtype):
    return synth.gaussian(shape, sigma, seed, dtype)


# ---------------------------------------------------------------- gemv
def test_gemv_config1_fp32():
    """1024 x 1024 fp32 weight N(0, 0.02^2), NF4 block 64, fp32 x and y."""
    W = synth.weight(1)
    x = synth.activations(1)
    packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4")
    y = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=torch.float32)
    p_ref, a_ref = O.quantize_4bit(f64(W), 64, "nf4")
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    check_matmul(f64(y), f64(x), w_hat(p_ref, a_ref, 1024, 1024, 64, "nf4"), "fp32", "fp32")


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_gemv_one_hot_returns_column_exactly(qt):
    N, K = 257, 2048
    W = gaussian((N, K), 0.02, 5, "fp32")
    p_ref, a_ref = O.quantize_4bit(f64(W), 64, qt)
    packed, st = upload_state(p_ref, a_ref, (N, K), torch.float32, 64, qt)
    What = O.dequantize_4bit(p_ref, a_ref, N * K, 64, qt).reshape(N, K)
    for k in (0, 31, 1000, K - 1):
        x = torch.zeros(1, K)
        x[0, k] = 1.0
        y = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=torch.float32).cpu().numpy()
        assert np.array_equal(y[0].view(np.uint32), What[:, k].view(np.uint32))


def test_gemv_config2_bf16():
    """4096 x 4096 bf16 weight, NF4 block 64, fp32 scales, bf16 x and y."""
    W = synth.weight(2)
    x = synth.activations(2)
    p_ref, a_ref = O.quantize_4bit(f64(W), 64, "nf4")
    packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4")
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    y = qmv.gemv_4bit(x.cuda(), packed, st)
    assert y.dtype == torch.bfloat16
    check_matmul(f64(y), f64(x), w_hat(p_ref, a_ref, 4096, 4096, 64, "nf4"), "bf16", "bf16")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("qt,dq", [("nf4", False), ("fp4", True)])
def test_gemv_all_m_ragged_n(M, qt, dq):
    N, K, bs = 333, 4096 + 512, 128
    W = gaussian((N, K), 0.02, 10 + M, "bf16")
    x = gaussian((M, K), 1.0, 20 + M, "bf16")
    p_ref, ahat = oracle_state(f64(W), bs, qt, dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, qt, double_quant=dq)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    y = qmv.gemv_4bit(x.cuda(), packed, st)
    Wh = w_hat(p_ref, ahat, N, K, bs, qt)
    check_matmul(f64(y), f64(x), Wh, "bf16", "bf16", f"M={M}")
    yf = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=torch.float32)
    check_matmul(f64(yf), f64(x), Wh, "bf16", "fp32", f"M={M} fp32 out")


@pytest.mark.parametrize("xd,yd", [("fp32", "fp32"), ("fp16", "fp16"), ("fp16", "fp32"),
                                   ("bf16", "fp32"), ("fp32", "bf16")])
def test_gemv_dtypes(xd, yd):
    N, K = 130, 1024
    W = gaussian((N, K), 0.02, 3, "bf16")
    x = gaussian((2, K), 1.0, 4, xd)
    p_ref, a_ref = O.quantize_4bit(f64(W), 64, "nf4")
    packed, st = upload_state(p_ref, a_ref, (N, K), torch.bfloat16, 64, "nf4")
    y = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=TDT[yd])
    check_matmul(f64(y), f64(x), w_hat(p_ref, a_ref, N, K, 64, "nf4"), xd, yd)


@pytest.mark.parametrize("bs", [32, 64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("dq", [False, True])
def test_matmul_all_blocksizes(bs, dq):
    """Every block size, including blocks longer than the 2048-weight slices
    the M = 1 kernels stream; K = 4096 + bs leaves a partial last slice."""
    N, K = 300, 4096 + bs
    W = gaussian((N, K), 0.02, bs + dq, "bf16")
    x = gaussian((5, K), 1.0, bs + 7, "bf16")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=dq)
    Wh = w_hat(p_ref, ahat, N, K, bs, "nf4")
    for M, f in ((1, qmv.gemv_4bit), (3, qmv.gemv_4bit), (5, qmv.gemm_4bit)):
        y = f(x[:M].contiguous().cuda(), packed, st, out_dtype=torch.float32)
        check_matmul(f64(y), f64(x[:M]), Wh, "bf16", "fp32", f"M={M} bs={bs} dq={dq}")


def test_gemv_m1_long_rows():
    """K = 49152: the activations are too long to stage in LDS, so the M = 1
    kernel reads them from global memory per slice."""
    N, K = 70, 49152
    W = gaussian((N, K), 0.02, 77, "bf16")
    x = gaussian((1, K), 1.0, 78, "bf16")
    for dq in (False, True):
        p_ref, ahat = oracle_state(f64(W), 64, "nf4", dq)
        packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4", double_quant=dq)
        y = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=torch.float32)
        check_matmul(f64(y), f64(x), w_hat(p_ref, ahat, N, K, 64, "nf4"), "bf16", "fp32")


def test_gemv_minimal_shapes():
    for N, K in ((1, 32), (5, 64), (64, 96)):
        W = gaussian((N, K), 0.02, N, "bf16")
        x = gaussian((1, K), 1.0, K, "fp32")
        p_ref, a_ref = O.quantize_4bit(f64(W), 32, "nf4")
        packed, st = upload_state(p_ref, a_ref, (N, K), torch.bfloat16, 32, "nf4")
        y = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=torch.float32)
        check_matmul(f64(y), f64(x), w_hat(p_ref, a_ref, N, K, 32, "nf4"), "fp32", "fp32")


# ---------------------------------------------------------------- gemm
@pytest.mark.parametrize("M", [1, 8, 100, 128, 300])
@pytest.mark.parametrize("qt,dq", [("nf4", False), ("fp4", True)])
def test_gemm_full_output(M, qt, dq):
    N, K, bs = 1000, 1024 + 64, 64
    W = gaussian((N, K), 0.02, 7, "bf16")
    A = gaussian((M, K), 1.0, 8, "bf16")
    p_ref, ahat = oracle_state(f64(W), bs, qt, dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, qt, double_quant=dq)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    C = qmv.gemm_4bit(A.cuda(), packed, st)
    Wh = w_hat(p_ref, ahat, N, K, bs, qt)
    check_matmul(f64(C), f64(A), Wh, "bf16", "bf16", f"M={M}")
    Cf = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=torch.float32)
    check_matmul(f64(Cf), f64(A), Wh, "bf16", "fp32", f"M={M} fp32 out")


@pytest.mark.parametrize("rows", [17, 32, 64, 200])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_gemm_identity_rows_exact(qt, rows):
    """Rows of the identity pick rows of the bf16 dequantized weight; every
    other product is an exact zero, so any order of summation is exact (17
    to 64 rows run the split-K kernel, 200 rows the tile kernel: both
    multiply bf16-rounded dequantized weights)."""
    N, K = 300, 256
    W = gaussian((N, K), 0.02, 9, "bf16")
    p_ref, a_ref = O.quantize_4bit(f64(W), 64, qt)
    packed, st = upload_state(p_ref, a_ref, (N, K), torch.bfloat16, 64, qt)
    A = torch.eye(K, dtype=torch.bfloat16)[:rows]
    C = qmv.gemm_4bit(A.cuda(), packed, st).cpu()
    What = O.dequantize_4bit(p_ref, a_ref, N * K, 64, qt, "bf16").reshape(N, K)
    got = C.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, What[:, :rows].T)


@pytest.mark.parametrize("rows", [1, 5, 8, 9, 16])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_gemm_narrow_identity_rows_exact(qt, rows):
    """Up to 16 rows and blocks of 64 or more take the narrow kernel, which
    multiplies bf16-rounded code values by the activations and applies the
    block scale per 64 k-values in fp32: a row of the identity then returns
    fp32(a_hat * bf16(T[code])) bit for bit (a zero of either sign reads +0,
    the sum of the other exact zeros), and its bf16 rounding."""
    N, K, bs = 300, 256, 64
    W = gaussian((N, K), 0.02, 19, "bf16")
    p_ref, a_ref = O.quantize_4bit(f64(W), bs, qt)
    packed, st = upload_state(p_ref, a_ref, (N, K), torch.bfloat16, bs, qt)
    A = torch.eye(K, dtype=torch.bfloat16)[3:3 + rows]
    t16 = O.f32_to_bf16_bits(O.code_table(qt).astype(np.float32)).astype(np.uint32) << np.uint32(16)
    codes = O.unpack_nibbles(p_ref, N * K).reshape(N, K)
    scale = np.repeat(a_ref.astype(np.float32).reshape(N, K // bs), bs, axis=1)
    w = t16.view(np.float32)[codes] * scale + np.float32(0)  # fp32 products, -0 -> +0
    want = np.ascontiguousarray(w[:, 3:3 + rows].T)
    C = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(C.view(np.uint32), want.view(np.uint32))
    Cb = qmv.gemm_4bit(A.cuda(), packed, st).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(Cb, O.f32_to_bf16_bits(want))


@pytest.mark.parametrize("M,N,K", [(5, 1000, 4096), (3, 8200, 4160), (6, 1000, 2048), (12, 2000, 2048),
                                   (16, 640, 8192), (8, 256, 1024)])
@pytest.mark.parametrize("dq", [False, True])
def test_gemm_narrow_many_waves(M, N, K, dq):
    """When the N / 32 workgroups leave compute units without a second one,
    the narrow kernel splits K over 8 or 16 waves per workgroup: 16 waves
    (8-row tile, 32 column groups with 32 groups of 128 k-values), 8 waves
    (8-row tile, 32 column groups with 16 k-groups; 16-row tile, 63 or 20
    column groups with 16 or 64 k-groups); 4 waves with more workgroups than
    compute units (257 workgroups, K = 4160 ending on half a group) and where
    K is too short to share (8 column groups with 8 k-groups)."""
    W = gaussian((N, K), 0.02, 3 * M + N + dq, "bf16")
    A = gaussian((M, K), 1.0, M + K + 1, "bf16")
    p_ref, ahat = oracle_state(f64(W), 64, "nf4", dq)
    packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4", double_quant=dq)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    Wh = w_hat(p_ref, ahat, N, K, 64, "nf4")
    for od in (torch.bfloat16, torch.float32):
        C = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=od)
        check_matmul(f64(C), f64(A), Wh, "bf16", od, f"M={M} N={N} K={K} dq={dq} {od}")
        if M <= 8:  # the gemv entry point takes the same kernel for 4 to 8 rows
            y = qmv.gemv_4bit(A.cuda(), packed, st, out_dtype=od)
            check_matmul(f64(y), f64(A), Wh, "bf16", od, f"gemv M={M} N={N} K={K} dq={dq} {od}")


@pytest.mark.parametrize("M", [1, 2, 8, 9, 16, 17, 31, 32, 33, 64, 65])
@pytest.mark.parametrize("K", [96, 192, 1600])
@pytest.mark.parametrize("dq", [False, True])
def test_gemm_skinny_ragged(M, K, dq):
    """Row counts around the row tiles of the split-K kernels (8, 16, 32 and
    64 rows; 65 is the first of the tile kernel).  N = 70 ends on a partial
    group of 32 output features.  K = 96 (block 32) is not a whole number of
    64-wide k-steps and takes the tile kernel; K = 192 leaves a wave with no
    k-step, K = 1600 gives the waves 7 or 6 steps each."""
    N, bs = 70, 32
    W = gaussian((N, K), 0.02, 40 + M, "bf16")
    A = gaussian((M, K), 1.0, 41 + M, "bf16")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", dq, bs2=32)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=dq, blocksize2=32)
    Wh = w_hat(p_ref, ahat, N, K, bs, "nf4")
    for od in (torch.float32, torch.bfloat16):
        C = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=od)
        assert C.shape == (M, N)
        check_matmul(f64(C), f64(A), Wh, "bf16", od, f"M={M} K={K} dq={dq} {od}")


def test_gemm_m1_matches_gemv():
    N, K = 4096, 4096
    W = gaussian((N, K), 0.02, 11, "bf16")
    x = gaussian((1, K), 1.0, 12, "bf16")
    packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4")
    y1 = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=torch.float32)
    y2 = qmv.gemm_4bit(x.cuda(), packed, st, out_dtype=torch.float32)
    # both within the bf16-activation bound of the same reference, so within
    # twice it of each other
    assert rel_l2(f64(y2), f64(y1)) <= 2 * (2.0 ** -8 + (K + 16) * 2.0 ** -24)


# ---------------------------------------------------------------- large M (128 x 256 tiles)
@pytest.mark.parametrize("M,N,K,bs", [(448, 2048, 192, 64), (500, 1000, 4160, 64), (777, 2080, 64, 32), (640, 3000, 1024, 128),
                                      (1030, 513, 1024, 64)])
@pytest.mark.parametrize("dq", [False, True])
def test_gemm_large_m_ragged(M, N, K, bs, dq):
    """M >= 448 takes the large-M kernel: a row tile past M (500, 777, 1030),
    column tiles past N (1000, 2080, 513; 2048 = 8 tiles of 256 takes the
    XCD-ordered mapping), a single k-tile (K = 64), 3 k-tiles, and K = 4160 =
    65 k-tiles (the loop's remainder path); blocks of 32, 64 and 128."""
    W = gaussian((N, K), 0.02, M + N + dq, "bf16")
    A = gaussian((M, K), 1.0, M + K, "bf16")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=dq)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    Wh = w_hat(p_ref, ahat, N, K, bs, "nf4")
    for od in (torch.bfloat16, torch.float32):
        C = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=od)
        assert C.shape == (M, N)
        check_matmul(f64(C), f64(A), Wh, "bf16", od, f"M={M} N={N} K={K} dq={dq} {od}")


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("xd", ["bf16", "fp16"])
def test_gemm_large_m_identity_rows_exact(qt, xd):
    """Rows of the identity among 600 rows of A: the large-M kernel multiplies
    fp32(T * a_hat) rounded to the activations' type, so those rows return the
    dequantize_4bit weights of that type bit for bit (a -0 weight reads +0);
    with a bias, one fp32 addition and one rounding."""
    M, N, K, bs = 600, 1000, 320, 64
    W = gaussian((N, K), 0.02, 61, "bf16")
    p_ref, a_ref = O.quantize_4bit(f64(W), bs, qt)
    packed, st = upload_state(p_ref, a_ref, (N, K), torch.bfloat16, bs, qt)
    A = gaussian((M, K), 1.0, 62, xd)
    rows = np.arange(100, 100 + K)            # rows 100 .. 419 are e_0 .. e_{K-1}
    A[torch.from_numpy(rows)] = 0
    A[torch.from_numpy(rows), torch.arange(K)] = 1
    C = qmv.gemm_4bit(A.cuda(), packed, st)
    got = C.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    want = np.asarray(O.dequantize_4bit(p_ref, a_ref, N * K, bs, qt, xd)).view(np.uint16).reshape(N, K).T.copy()
    zero = 0x8000
    want[want == zero] = 0
    got = got.copy()
    got[got == zero] = 0
    assert np.array_equal(got, want)
    bias = gaussian((N,), 0.5, 63, xd).cuda()
    Cf = qmv.gemm_4bit(A.cuda(), packed, st, out_dtype=torch.float32)
    Cb = qmv.gemm_4bit(A.cuda(), packed, st, bias=bias)
    assert torch.equal(Cb.cpu(), (Cf + bias.float()).to(Cb.dtype).cpu())
    Wh = w_hat(p_ref, a_ref, N, K, bs, qt)
    check_matmul(f64(Cf), f64(A), Wh, xd, "fp32", f"{qt} {xd} fp32 out")
