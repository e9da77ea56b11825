"""GPU parity of the gemv kernel for 1 to 4 activation rows (the decode step
and small batches) on every way it can be launched: activations held in
registers (up to 4 slices of 2048 weights per row, over all rows), read per
slice from the staged LDS copy, or read from global memory (longer rows);
partial last slices; more rows than waves (some waves carry one extra row)
and fewer rows than waves (some carry none).
Reference: the CPU oracle's dequantize + float64 matmul, compared by
``bounds.check_matmul`` (relative L2 over the whole output and the derived
per-element bound)."""
import numpy as np
import pytest
import torch

import oracle as O
from bounds import check_matmul
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()



CASES = [
    # (N, K, blocksize, dq): what the case reaches
    (4873, 1024, 64, True),     # one half-filled slice per row; rows % waves != 0
    (333, 2080, 32, False),     # second slice holds a single 16-byte piece
    (1500, 6208, 64, True),     # four slices in registers, the last one partial
    (700, 10368, 128, True),    # six slices: activations read from LDS per slice
    (100, 4096, 64, True),      # fewer rows than waves: most waves have no row
    (1, 4096, 64, False),       # a single row
    (9, 6144, 2048, True),      # three slices per row, one block per slice
    (4101, 8256, 64, True),     # activations from LDS, rows taken in pairs on the waves with two
    (12290, 8224, 32, False),   # three rows per wave: the last one paired with a dead row
]


@pytest.mark.parametrize("N,K,bs,dq", CASES)
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_gemv_m1_paths(N, K, bs, dq, qt):
    seed = N * 7 + K + bs + dq
    W = synth.gaussian((N, K), 0.02, seed, "bf16")
    p_ref, absmax = O.quantize_4bit(f64(W), bs, qt)
    if dq:
        q, a2, off = O.double_quant(absmax, 256)
        ahat = O.dequant_absmax(q, a2, off, None, 256)
    else:
        ahat = absmax
    packed, st = qmv.quantize_4bit(W.cuda(), bs, qt, double_quant=dq)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    Wh = O.dequantize_4bit(p_ref, ahat, N * K, bs, qt).reshape(N, K)
    for M in (1, 2, 3, 4):
        xm = synth.gaussian((M, K), 1.0, seed + 1 + M, "bf16")
        yf = qmv.gemv_4bit(xm.cuda(), packed, st, out_dtype=torch.float32)
        assert yf.shape == (M, N)
        assert np.all(np.isfinite(f64(yf)))
        check_matmul(f64(yf), f64(xm), Wh, "bf16", "fp32", f"M={M} fp32 out")
        yb = qmv.gemv_4bit(xm.cuda(), packed, st)
        check_matmul(f64(yb), f64(xm), Wh, "bf16", "bf16", f"M={M} bf16 out")


def test_gemv_m1_repeatable():
    """Two launches give the same bits (no cross-wave accumulation order)."""
    N, K = 14336 // 4, 4096
    W = synth.gaussian((N, K), 0.02, 5, "bf16").cuda()
    x = synth.gaussian((1, K), 1.0, 6, "bf16").cuda()
    packed, st = qmv.quantize_4bit(W, 64, "nf4", double_quant=True)
    y1 = qmv.gemv_4bit(x, packed, st, out_dtype=torch.float32)
    y2 = qmv.gemv_4bit(x, packed, st, out_dtype=torch.float32)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("M,odt", [(1, "fp32"), (3, "bf16")])
def test_gemv_m1_long_runs_with_bias(M, odt):
    """More than 64 rows per wave (64 * 4096 + 100 rows): the bias of rows past
    a run's 64th is read per row instead of from the read-ahead copy (fp32
    and 16-bit bias, which take different loads)."""
    N, K, bs = 64 * 4096 + 100, 64, 64
    W = synth.gaussian((N, K), 0.02, 91, "bf16")
    x = synth.gaussian((M, K), 1.0, 92, "bf16")
    bias = synth.gaussian((N,), 0.1, 93, odt)
    p_ref, absmax = O.quantize_4bit(f64(W), bs, "nf4")
    packed, st = qmv.quantize_4bit(W.cuda(), bs, "nf4")
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    Wh = O.dequantize_4bit(p_ref, absmax, N * K, bs, "nf4").reshape(N, K)
    y = qmv.gemv_4bit(x.cuda(), packed, st, out_dtype=TDT[odt], bias=bias.cuda())
    check_matmul(f64(y), f64(x), Wh, "bf16", odt, "all rows", bias=f64(bias))
    # the rows past each run's 64th, checked on their own
    runs = 4096
    rpw, rem = N // runs, N % runs
    starts = np.array([r * rpw + min(r, rem) for r in range(runs)])
    late = (starts[:, None] + np.arange(64, rpw + 1)[None, :]).reshape(-1)
    late = late[late < N]
    check_matmul(f64(y)[:, late], f64(x), Wh[late], "bf16", odt, "late rows", bias=f64(bias)[late])
