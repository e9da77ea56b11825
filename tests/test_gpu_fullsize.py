"""Parity at the full workload sizes: the 1024 x 1024 fp32 and 4096 x 4096
bf16 round trips with gemv, the 14336 x 4096 / 4096 x 14336 MLP
weights (NF4 and FP4, block 64, double-quantized scales, gemv M = 1), the
gemm prefill shapes (M in 8, 32, 128, 512 on the 14336 x 4096 NF4 weight),
and the 8192 x 28672 / 28672 x 8192 layers (block 128, double-quantized,
dequantize to bf16, gemv M in 1, 2, 4, 8).

Everything runs through the same Python entry points, and therefore the same
kernels and launch shapes, that bench.py times.  The oracle is too slow for
whole tensors, so it recomputes a sample of rows one by one: the packed codes
and scales of those rows and their dequantized bf16 values must be bit-exact,
and the matmul outputs of those output features must be within the relative
L2 tolerance (2e-2 for bf16 outputs).  Block scales and the double-quant state
are cheap and are compared in full."""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def bits32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


@functools.lru_cache(maxsize=2)
def weight_cpu(cfg, which):
    return synth.weight(cfg, which)


@functools.lru_cache(maxsize=2)
def oracle_absmax(cfg, which):
    W = weight_cpu(cfg, which)
    bs = synth.WORKLOADS[cfg].blocksize
    return O.block_absmax(W.to(torch.float32).numpy(), bs).astype(np.float32)


def sample_rows(N, seed, n=40):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, n, replace=False)]))


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def run_case(cfg, which, qt, ms, matmul, extra_gemm=()):
    wl = synth.WORKLOADS[cfg]
    N, K = wl.weights[which]
    bs = wl.blocksize
    W_cpu = weight_cpu(cfg, which)
    print(f"[fullsize] workload {cfg} weight {which} {N}x{K} {qt} bs{bs} dq={wl.double_quant}",
          flush=True)
    packed, st = qmv.quantize_4bit(W_cpu.cuda(), bs, qt)
    if wl.double_quant:
        q, a2, off, c2 = qmv.double_quant(st.absmax, 256)
        st_use = qmv.QuantState(st.shape, st.dtype, bs, qt, None, q, a2, off, c2, 256)
    else:
        st_use = st
    torch.cuda.synchronize()

    # block scales in full
    a_ref = oracle_absmax(cfg, which)
    assert np.array_equal(bits32(st.absmax.cpu().numpy()), bits32(a_ref))
    if wl.double_quant:
        q_ref, a2_ref, off_ref = O.double_quant(a_ref, 256)
        assert bits32(off.cpu().numpy())[0] == bits32([off_ref])[0]
        assert np.array_equal(bits32(a2.cpu().numpy()), bits32(a2_ref))
        assert np.array_equal(q.cpu().numpy(), q_ref)
        ahat = O.dequant_absmax(q_ref, a2_ref, off_ref)
    else:
        ahat = a_ref

    # sampled rows: codes, then dequantized values
    rows = sample_rows(N, seed=1000 * cfg + 10 * which + (qt == "fp4"))
    W64 = W_cpu[torch.from_numpy(rows)].to(torch.float64).numpy()
    p_rows, a_rows = O.quantize_4bit(W64, bs, qt)
    assert np.array_equal(bits32(a_rows), bits32(a_ref.reshape(N, K // bs)[rows].ravel()))
    got_p = packed.view(N, K // 2)[torch.from_numpy(rows).cuda()].cpu().numpy().ravel()
    bad = np.flatnonzero(got_p != p_rows)
    assert bad.size == 0, f"{bad.size} packed bytes differ in the sampled rows"
    ahat_rows = ahat.reshape(N, K // bs)[rows].ravel()
    w_rows = O.dequantize_4bit(p_rows, ahat_rows, rows.size * K, bs, qt)      # fp32
    w_bf16 = qmv.dequantize_4bit(packed, st_use, out_dtype=torch.bfloat16)
    got_w = w_bf16[torch.from_numpy(rows).cuda()].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_w.ravel(), O.f32_to_bf16_bits(w_rows))
    del w_bf16

    # matmul outputs of the sampled output features
    Wr = w_rows.reshape(rows.size, K).astype(np.float64)
    for M, kind in [(m, matmul) for m in ms] + [(m, "gemm") for m in extra_gemm]:
        # the prefill activations of workload 4 (prefix-stable in M)
        x = synth.activations(4 if kind == "gemm" else cfg, which if kind == "gemv" else 0, M)
        f = qmv.gemv_4bit if kind == "gemv" else qmv.gemm_4bit
        y = f(x.cuda(), packed, st_use)
        torch.cuda.synchronize()
        assert y.dtype == x.dtype and y.shape == (M, N)
        tol = 1e-3 if y.dtype == torch.float32 else BF16_TOL
        got = y[:, torch.from_numpy(rows).cuda()].cpu().to(torch.float64).numpy()
        ref = x.to(torch.float64).numpy() @ Wr.T
        err = rel_l2(got, ref)
        print(f"[fullsize]   {kind} M={M}: sampled rel-L2 {err:.2e}", flush=True)
        assert err <= tol, (M, err)


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
