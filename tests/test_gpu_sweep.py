"""Randomized GPU parity sweep: seeded random shapes, block sizes, code
types, scale kinds, activation / output dtypes and bias, each case checked
end to end against the CPU oracle (quantize bit for bit, then the matmuls
within the tolerances of the fixed-shape tests).  Every case draws its
parameters from its own seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import oracle as O
from bounds import check_backward, check_matmul
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
N_CASES = 120


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def draw(i):
    rng = np.random.default_rng(1000 + i)
    bs = int(rng.choice([32, 64, 128, 256]))
    K = bs * int(rng.integers(1, max(2, 1024 // bs) + 1))
    if K % 32:
        K += 32 - K % 32
    N = int(rng.integers(1, 320)) if rng.integers(0, 2) else 32 * int(rng.integers(1, 10))
    return dict(
        bs=bs, K=K, N=N,
        qt=str(rng.choice(["nf4", "fp4"])),
        dq=bool(rng.integers(0, 2)),
        bs2=int(rng.choice([32, 64, 256])),
        wdt=str(rng.choice(["bf16", "fp16", "fp32"])),
        xdt=str(rng.choice(["bf16", "fp16", "fp32"])),
        odt=str(rng.choice(["bf16", "fp16", "fp32"])),
        M_gemv=int(rng.integers(1, 9)),
        M_gemm=int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 300))])),
        bias=bool(rng.integers(0, 2)),
        seed=int(rng.integers(0, 1 << 30)),
    )


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i):
    c = draw(i)
    N, K, bs, qt, dq = c["N"], c["K"], c["bs"], c["qt"], c["dq"]
    W = synth.gaussian((N, K), 0.02, c["seed"], c["wdt"])
    packed, st = qmv.quantize_4bit(W.cuda(), bs, qt, double_quant=dq, blocksize2=c["bs2"])
    p_ref, a_ref = O.quantize_4bit(f64(W), bs, qt)
    assert np.array_equal(packed.cpu().numpy(), p_ref), c
    if dq:
        q, a2, off = O.double_quant(a_ref, c["bs2"])
        ahat = O.dequant_absmax(q, a2, off, None, c["bs2"])
        assert np.array_equal(st.absmax_q.cpu().numpy(), q), c
    else:
        ahat = a_ref
    # dequantize, bit for bit
    w = qmv.dequantize_4bit(packed, st, out_dtype=torch.float32).cpu().numpy().reshape(-1)
    w_ref = O.dequantize_4bit(p_ref, ahat, N * K, bs, qt)
    assert np.array_equal(w.view(np.uint32), w_ref.view(np.uint32)), c

    bias = synth.gaussian((N,), 0.1, c["seed"] + 1, c["odt"]).cuda() if c["bias"] else None
    b64 = f64(bias) if bias is not None else None
    Wh = w_ref.reshape(N, K)
    for M, f in ((c["M_gemv"], qmv.gemv_4bit), (c["M_gemm"], qmv.gemm_4bit)):
        x = synth.gaussian((M, K), 1.0, c["seed"] + 2 + M, c["xdt"])
        y = f(x.cuda(), packed, st, out_dtype=TDT[c["odt"]], bias=bias)
        assert y.shape == (M, N)
        check_matmul(f64(y), f64(x), Wh, c["xdt"], c["odt"], f"{c} M={M} {f.__name__}", bias=b64)

    # backward (16-bit dY, N a multiple of 32)
    if c["xdt"] != "fp32" and N % 32 == 0:
        M = c["M_gemm"]
        dY = synth.gaussian((M, N), 1.0, c["seed"] + 3, c["xdt"])
        dX = qmv.gemm_4bit_backward(dY.cuda(), packed, st, out_dtype=TDT[c["odt"]])
        check_backward(f64(dX), f64(dY), Wh, c["xdt"], c["odt"], f"{c} backward")
