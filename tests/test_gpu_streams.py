"""Stream ordering through the C ABI.  Every entry point takes a stream and
only enqueues on it ("Feat/mps gemm 4bit bf16", "Performance": the pages'
design pays two host synchronizations per native call; this library pays
none).  The Python layer passes torch's current stream.

A side stream is held behind a long chain of matrix products; then, on that
stream and with no host synchronization anywhere, each iteration writes a
fresh weight with a torch op (the base weight times its own power of two,
so each iteration's block scales differ) and runs quantize_4bit -> double quant ->
gemv_4bit -> gemm_4bit on it.  The test has teeth both ways:
* if a call ran on another stream (or the null stream), it would read the
  weight before the producer wrote it (the buffer holds zeros or another
  iteration's values) and its outputs would not match the oracle;
* if a call synchronized the host or the device, the side stream's work
  would already be complete when the enqueueing returns.
Checks: right after enqueueing, and again after synchronizing the null
stream only, the side stream's event is not complete; after waiting on it,
every iteration's outputs equal the oracle's (bit for bit for the codes and
scales, within the derived bounds for the matmuls)."""
import numpy as np
import pytest
import torch

import oracle as O
from bounds import check_matmul
from quantized_matvec_amd import qmv, synth

pytestmark = pytest.mark.gpu
ITERS = 24
N, K, BS = 384, 1024, 64


def test_side_stream_ordering_without_host_sync():
    dev = torch.device("cuda")
    base = synth.gaussian((N, K), 0.02, 777, "bf16").to(dev)
    x = synth.gaussian((1, K), 1.0, 778, "bf16").to(dev)
    A = synth.gaussian((40, K), 1.0, 779, "bf16").to(dev)
    big = torch.randn(4096, 4096, device=dev)
    torch.cuda.synchronize()

    side = torch.cuda.Stream(device=dev)
    outs = []
    with torch.cuda.stream(side):
        h = big
        for _ in range(120):                        # over 100 ms of work ahead
            h = torch.tanh(h @ big) * 0.01
        for i in range(ITERS):
            W = torch.zeros(N, K, dtype=torch.bfloat16, device=dev)
            torch.mul(base, 2.0 ** (i - 12), out=W)         # the producer: exact in bf16
            packed, st = qmv.quantize_4bit(W, BS, "nf4", double_quant=True)
            y = qmv.gemv_4bit(x, packed, st, out_dtype=torch.float32)
            C = qmv.gemm_4bit(A, packed, st, out_dtype=torch.float32)
            outs.append((packed, st, y, C))
        done = torch.cuda.Event()
        done.record(side)
    assert not done.query(), "the side stream finished while it was being fed: something synchronized"
    torch.cuda.default_stream(dev).synchronize()
    assert not done.query(), "synchronizing the null stream waited for the side stream's work"
    done.synchronize()
    _ = h.sum().item()

    for i, (packed, st, y, C) in enumerate(outs):
        Wi = (base.cpu().to(torch.float64) * 2.0 ** (i - 12)).numpy()
        p_ref, a_ref = O.quantize_4bit(Wi, BS, "nf4")
        q, a2, off = O.double_quant(a_ref, 256)
        assert np.array_equal(packed.cpu().numpy(), p_ref), i
        assert np.array_equal(st.absmax_q.cpu().numpy(), q), i
        assert np.array_equal(st.absmax2.cpu().numpy().view(np.uint32), a2.view(np.uint32)), i
        assert np.float32(st.offset.item()) == off, i
        ahat = O.dequant_absmax(q, a2, off)
        Wh = O.dequantize_4bit(p_ref, ahat, N * K, BS, "nf4").reshape(N, K)
        check_matmul(y.cpu().double().numpy(), x.cpu().double().numpy(), Wh, "bf16", "fp32", f"gemv {i}")
        check_matmul(C.cpu().double().numpy(), A.cpu().double().numpy(), Wh, "bf16", "fp32", f"gemm {i}")
