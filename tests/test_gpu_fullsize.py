"""Parity at the full workload sizes, over whole tensors: the 1024 x 1024 fp32
and 4096 x 4096 bf16 round trips with gemv, the 14336 x 4096 / 4096 x 14336
MLP weights (NF4 and FP4, block 64, double-quantized scales, gemv M = 1), the
gemm prefill shapes (M in 8, 32, 128, 512 on the 14336 x 4096 NF4 weight;
also 1024 and 2048), and the 8192 x 28672 / 28672 x 8192 layers (block 128,
double-quantized, dequantize to bf16, gemv M in 1, 2, 4, 8).

Everything runs through the same Python entry points, and therefore the same
kernels and launch shapes, that bench.py times.  The oracle quantizes each
whole weight with its threshold form (the literal 16-distance form is pinned
equal to it on smaller inputs) and everything is compared in full: every
packed byte, every block scale, the double-quant state, every bf16 weight of
dequantize_4bit, and every matmul output (relative L2 over all outputs plus
the per-element bound of ``bounds.check_matmul``).  At these sizes
quantize_4bit and dequantize_4bit walk many tiles per workgroup, so their
grid-stride loops and double-buffered stages run here."""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from bounds import check_matmul
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu


def bits32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def assert_equal_bytes(got, want, what):
    got = np.asarray(got).ravel()
    want = np.asarray(want).ravel()
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} of {want.size} differ, first at {bad[:6]}"


@functools.lru_cache(maxsize=1)
def weight_cpu(cfg, which):
    return synth.weight(cfg, which)


@functools.lru_cache(maxsize=1)
def oracle_state(cfg, which, qt):
    """The oracle's quantization of the whole weight (threshold form)."""
    wl = synth.WORKLOADS[cfg]
    W = weight_cpu(cfg, which)
    x = W.to(torch.float64).numpy()
    packed, absmax = O.quantize_4bit(x, wl.blocksize, qt, forms="threshold")
    st = {"packed": packed, "absmax": absmax}
    if wl.double_quant:
        q, a2, off = O.double_quant(absmax, 256, forms="threshold")
        st.update(q=q, absmax2=a2, offset=off, ahat=O.dequant_absmax(q, a2, off))
    else:
        st["ahat"] = absmax
    return st


def run_case(cfg, which, qt, ms, kind, extra_gemm=()):
    wl = synth.WORKLOADS[cfg]
    N, K = wl.weights[which]
    bs = wl.blocksize
    print(f"[fullsize] workload {cfg} weight {which} {N}x{K} {qt} bs{bs} dq={wl.double_quant}",
          flush=True)
    W_cpu = weight_cpu(cfg, which)
    packed, st = qmv.quantize_4bit(W_cpu.cuda(), bs, qt)
    if wl.double_quant:
        q, a2, off, c2 = qmv.double_quant(st.absmax, 256)
        st_use = qmv.QuantState(st.shape, st.dtype, bs, qt, None, q, a2, off, c2, 256)
    else:
        st_use = st
    torch.cuda.synchronize()
    ref = oracle_state(cfg, which, qt)

    # the codec, whole tensors, bit for bit
    assert_equal_bytes(packed.cpu().numpy(), ref["packed"], "packed codes")
    assert_equal_bytes(bits32(st.absmax.cpu().numpy()), bits32(ref["absmax"]), "block absmax")
    if wl.double_quant:
        assert bits32(off.cpu().numpy())[0] == bits32([ref["offset"]])[0], "double-quant offset"
        assert_equal_bytes(bits32(a2.cpu().numpy()), bits32(ref["absmax2"]), "group scales")
        assert_equal_bytes(q.cpu().numpy(), ref["q"], "8-bit scale codes")
    w_ref = O.dequantize_4bit(ref["packed"], ref["ahat"], N * K, bs, qt)          # fp32
    out_dt = torch.float32 if wl.w_dtype == "fp32" else torch.bfloat16
    w_gpu = qmv.dequantize_4bit(packed, st_use, out_dtype=out_dt)
    if out_dt == torch.float32:
        assert_equal_bytes(bits32(w_gpu.cpu().numpy()), bits32(w_ref), "fp32 dequantized weights")
    else:
        got = w_gpu.cpu().view(torch.int16).numpy().view(np.uint16)
        assert_equal_bytes(got, O.f32_to_bf16_bits(w_ref), "bf16 dequantized weights")
    del w_gpu
    print(f"[fullsize]   codec bit-exact over {N * K} weights", flush=True)

    # the matmuls, every output
    Wh = w_ref.reshape(N, K).astype(np.float64)
    del w_ref
    for M, k in [(m, kind) for m in ms] + [(m, "gemm") for m in extra_gemm]:
        # the prefill activations of workload 4 (prefix-stable in M)
        x = synth.activations(4 if k == "gemm" else cfg, which if k == "gemv" else 0, M)
        f = qmv.gemv_4bit if k == "gemv" else qmv.gemm_4bit
        y = f(x.cuda(), packed, st_use)
        torch.cuda.synchronize()
        assert y.dtype == x.dtype and y.shape == (M, N)
        err = check_matmul(y.cpu().to(torch.float64).numpy(), x.to(torch.float64).numpy(), Wh,
                           x.dtype, y.dtype, f"{k} M={M}")
        print(f"[fullsize]   {k} M={M}: rel-L2 {err:.2e} over all {M * N} outputs", flush=True)


@pytest.mark.parametrize("cfg", [1, 2])
def test_small_layers_round_trip_gemv(cfg):
    """1024 x 1024 fp32 (fp32 x and y) and 4096 x 4096 bf16, NF4, block 64."""
    run_case(cfg, 0, "nf4", (1,), "gemv")


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("which", [0, 1])
def test_mlp_layers_gemv_m1(which, qt):
    """14336 x 4096 and 4096 x 14336, block 64, double-quantized, M = 1; on the
    14336 x 4096 NF4 weight also gemm at M = 512 (the step bench.py times)."""
    run_case(3, which, qt, (1,), "gemv", (512,) if (which, qt) == (0, "nf4") else ())


def test_gemm_prefill_shapes():
    """14336 x 4096 NF4, block 64, A bf16 [M, 4096], M in 8, 32, 128, 512."""
    run_case(4, 0, "nf4", (8, 32, 128, 512), "gemm")


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("which", [0, 1])
def test_large_layers_gemv_m1_to_8(which, qt):
    """8192 x 28672 and 28672 x 8192, block 128, double-quantized, M in 1, 2, 4, 8."""
    run_case(5, which, qt, (1, 2, 4, 8), "gemv")


@pytest.mark.parametrize("M", [1024, 2048])
def test_gemm_beyond_512_rows(M):
    """gemm above the prefill shapes (the pull-request page measures M up to
    2048): the 14336 x 4096 NF4 weight with A [M, 4096] bf16, buffers sized
    for M rows.  Every row is compared on 512 sampled output columns (plus the
    first and last), and 64 rows of A are rows of the identity, which must
    return the bf16 dequantized weight columns bit for bit."""
    N, K = synth.WORKLOADS[4].weights[0]
    W_cpu = weight_cpu(4, 0)
    A = synth.gaussian((M, K), 1.0, 4000 + M, "bf16")
    eye_rows = np.arange(M // 2, M // 2 + 64)
    eye_cols = np.random.default_rng(M).choice(K, 64, replace=False)
    A[torch.from_numpy(eye_rows)] = 0
    A[torch.from_numpy(eye_rows), torch.from_numpy(eye_cols)] = 1
    packed, st = qmv.quantize_4bit(W_cpu.cuda(), 64, "nf4")
    C = qmv.gemm_4bit(A.cuda(), packed, st)
    torch.cuda.synchronize()
    assert C.shape == (M, N)
    ref = oracle_state(4, 0, "nf4")
    assert_equal_bytes(packed.cpu().numpy(), ref["packed"], "packed codes")
    cols = np.unique(np.concatenate([[0, N - 1],
                                     np.random.default_rng(M + 1).choice(N, 512, replace=False)]))
    W_hat = O.dequantize_4bit(ref["packed"], ref["ahat"], N * K, 64, "nf4").reshape(N, K)
    Wc = W_hat[cols].astype(np.float64)
    got = C[:, torch.from_numpy(cols).cuda()].cpu().to(torch.float64).numpy()
    err = check_matmul(got, A.to(torch.float64).numpy(), Wc, "bf16", "bf16", f"gemm M={M}")
    print(f"[fullsize] gemm M={M}: rel-L2 {err:.2e} on {cols.size} columns of every row", flush=True)
    # identity rows: C[r, n] = bf16(W_hat[n, k_r]) exactly, every column
    want = O.f32_to_bf16_bits(np.ascontiguousarray(W_hat[:, eye_cols].T))
    got_i = C[torch.from_numpy(eye_rows).cuda()].cpu().view(torch.int16).numpy().view(np.uint16)
    want[want == 0x8000] = 0   # a -0 weight reads +0 (the sum of the other exact zeros)
    got_i = got_i.copy()
    got_i[got_i == 0x8000] = 0
    assert_equal_bytes(got_i, want, "identity rows")
