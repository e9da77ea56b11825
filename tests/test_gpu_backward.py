"""GPU parity of gemm_4bit_backward (dX = dY @ W_hat) against the CPU oracle
(the composition grad_output @ dequantize_4bit(B), in float64), through the
C ABI.

Compared by ``bounds.check_backward``: relative L2 over all of dX and the
derived per-element bound (the contraction runs over N).  Exact pin: rows of
the identity as dY return rows of the bf16 dequantized weight bit for bit.
Full size: the 14336 x 4096 NF4 weight of the MLP workload with a 512-row
gradient."""
import numpy as np
import pytest
import torch

import oracle as O
from bounds import check_backward
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def oracle_state(W64, bs, qt, dq, bs2=256):
    packed, absmax = O.quantize_4bit(W64, bs, qt)
    if dq:
        q, a2, off = O.double_quant(absmax, bs2)
        return packed, O.dequant_absmax(q, a2, off, None, bs2)
    return packed, absmax


@pytest.mark.parametrize("M,N,K,bs", [(1, 64, 64, 64), (5, 96, 192, 32), (128, 992, 1088, 64),
                                      (130, 320, 256, 128), (300, 64, 4160, 64)])
@pytest.mark.parametrize("qt,dq", [("nf4", False), ("fp4", True)])
def test_backward_shapes(M, N, K, bs, qt, dq):
    """Ragged M (row tiles of 128), N = 96 and 992 end on half a 64-row step,
    K = 1088 and 4160 on a partial column tile; narrow (64-column) and wide
    tiles both run."""
    W = synth.gaussian((N, K), 0.02, 3 * N + K, "bf16")
    dY = synth.gaussian((M, N), 1.0, 7 * M + N, "bf16")
    p_ref, ahat = oracle_state(f64(W), bs, qt, dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, qt, double_quant=dq)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    Wh = O.dequantize_4bit(p_ref, ahat, N * K, bs, qt).reshape(N, K)
    for od in (torch.bfloat16, torch.float32):
        dX = qmv.gemm_4bit_backward(dY.cuda(), packed, st, out_dtype=od)
        assert dX.shape == (M, K) and dX.dtype == od
        check_backward(f64(dX), f64(dY), Wh, "bf16", od, f"{(M, N, K, od)}")


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_backward_identity_rows_exact(qt):
    """dY = rows of the identity: dX row i is weight row i, dequantized to
    bf16 (fp32(T * a_hat) rounded), bit for bit; every other product is an
    exact zero."""
    N, K, bs = 192, 320, 64
    W = synth.gaussian((N, K), 0.02, 21, "bf16")
    p_ref, a_ref = O.quantize_4bit(f64(W), bs, qt)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, qt)
    dY = torch.eye(N, dtype=torch.bfloat16)[5:5 + 150]
    dX = qmv.gemm_4bit_backward(dY.cuda(), packed, st).cpu()
    What = O.dequantize_4bit(p_ref, a_ref, N * K, bs, qt, "bf16").reshape(N, K)
    got = dX.view(torch.int16).numpy().view(np.uint16)
    # a -0 weight reads as +0 (the sum of the other exact zeros)
    want = What[5:5 + 150].copy()
    want[want == 0x8000] = 0
    got = got.copy()
    got[got == 0x8000] = 0
    assert np.array_equal(got, want)


def test_backward_full_size_sampled():
    """W_up 14336 x 4096 NF4 (block 64, double-quantized scales) with a
    512-row bf16 gradient that is non-zero on 66 sampled weight rows only, so
    that the oracle quantizes just those rows (the double-quant mean still
    comes from every block): all of dX is compared, every tile runs."""
    N, K = synth.WORKLOADS[3].weights[0]
    W = synth.weight(3, 0)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(5).choice(N, 64, replace=False)]))
    dY = torch.zeros((512, N), dtype=torch.bfloat16)
    dY[:, torch.from_numpy(rows)] = synth.gaussian((512, rows.size), 1.0, 99, "bf16")
    packed, st = qmv.quantize_4bit(W.cuda(), 64, "nf4", double_quant=True)
    dX = qmv.gemm_4bit_backward(dY.cuda(), packed, st)
    torch.cuda.synchronize()
    a_full = O.block_absmax(W.to(torch.float32).numpy(), 64).astype(np.float32)
    q, a2, off = O.double_quant(a_full, 256)
    ahat = O.dequant_absmax(q, a2, off).reshape(N, K // 64)[rows].ravel()
    p_rows, _ = O.quantize_4bit(W[torch.from_numpy(rows)].to(torch.float64).numpy(), 64, "nf4")
    Wh = O.dequantize_4bit(p_rows, ahat, rows.size * K, 64, "nf4").reshape(rows.size, K)
    err = check_backward(f64(dX), f64(dY[:, torch.from_numpy(rows)]), Wh, "bf16", "bf16", "full size")
    print(f"[backward] full size, sampled rows: rel-L2 {err:.2e}", flush=True)
