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


@pytest.mark.parametrize("M,N,K,bs", [(130, 320, 256, 128), (256, 640, 512, 64), (1000, 1024, 1024, 64),
                                      (2048, 384, 2048, 256), (2048, 256, 4096, 64)])
@pytest.mark.parametrize("dq", [False, True])
def test_backward_split_reduction(M, N, K, bs, dq):
    """Shapes the transposed-read kernel takes (N % 64 == 0, K % 256 == 0,
    blocks of 64 or more): its reduction split over 5, 10, 8, 2 and 1
    workgroups per 128 x 256 tile (one to three steps of 64 rows each, and
    ragged row tiles at M = 130 and 1000).  Compared with the oracle, and
    repeated: the splits are added in a fixed order, so a second call gives
    the same bits.  The shapes run in one workspace, so a call's tile
    counters sit where an earlier shape left partial sums."""
    W = synth.gaussian((N, K), 0.02, 5 * N + K, "bf16")
    dY = synth.gaussian((M, N), 1.0, 11 * M + N, "bf16")
    p_ref, ahat = oracle_state(f64(W), bs, "nf4", dq)
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4", double_quant=dq)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    Wh = O.dequantize_4bit(p_ref, ahat, N * K, bs, "nf4").reshape(N, K)
    print(f"[backward] split path {(M, N, K, bs, dq)}", flush=True)
    for od in (torch.bfloat16, torch.float32):
        d1 = qmv.gemm_4bit_backward(dY.cuda(), packed, st, out_dtype=od)
        d2 = qmv.gemm_4bit_backward(dY.cuda(), packed, st, out_dtype=od)
        assert torch.equal(d1.view(torch.int16) if od != torch.float32 else d1.view(torch.int32),
                           d2.view(torch.int16) if od != torch.float32 else d2.view(torch.int32))
        check_backward(f64(d1), f64(dY), Wh, "bf16", od, f"{(M, N, K, od)}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_backward_split_identity_rows_exact(dt):
    """The transposed-read kernel with dY = rows of the identity returns the
    weight rows as dequantize_4bit gives them in dY's type, bit for bit: the
    transposition moves every decoded value to the right place, and the
    split reduction adds only exact zeros to it."""
    N, K, bs = 256, 512, 64
    W = synth.gaussian((N, K), 0.02, 23, "bf16")
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "fp4", double_quant=True)
    want = qmv.dequantize_4bit(packed, st, out_dtype=dt).cpu().view(torch.int16).numpy().view(np.uint16)
    dY = torch.eye(N, dtype=dt)[3:3 + 200]
    got = qmv.gemm_4bit_backward(dY.cuda(), packed, st).cpu().view(torch.int16).numpy().view(np.uint16).copy()
    want = want[3:3 + 200].copy()
    sign0 = 0x8000
    want[want == sign0] = 0
    got[got == sign0] = 0
    assert np.array_equal(got, want)


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
