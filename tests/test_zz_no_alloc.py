"""qmv_double_quant_noalloc (no workspace, no allocation; its scratch is a
fixed array the library keeps on each GPU) against qmv_double_quant with a
caller workspace: bit for bit on consecutive calls, each smaller than the one
before, so the fixed scratch still holds the previous call's partial sums
when the next call starts.  Both are called through the C ABI."""
import numpy as np
import pytest
import torch

import crafted_inputs
from quantized_matvec_amd import qmv

pytestmark = pytest.mark.gpu


def call(a, bs2, noalloc):
    L = qmv.lib()
    n = a.numel()
    dev = a.device
    q = torch.full((n,), 0xAB, dtype=torch.uint8, device=dev)
    a2 = torch.full((-(-n // bs2),), -1.0, dtype=torch.float32, device=dev)
    off = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
    c2 = torch.zeros(256, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        rc = L.qmv_double_quant_noalloc(a.data_ptr(), n, bs2, None, q.data_ptr(), a2.data_ptr(),
                                        off.data_ptr(), c2.data_ptr(), st)
    else:
        ws = torch.empty(L.qmv_double_quant_workspace(n, bs2), dtype=torch.uint8, device=dev)
        rc = L.qmv_double_quant(a.data_ptr(), n, bs2, None, q.data_ptr(), a2.data_ptr(),
                                off.data_ptr(), c2.data_ptr(), ws.data_ptr(), ws.numel(), st)
    assert rc == 0, qmv.STATUS.get(rc, rc)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (q, a2, off, c2)]


def scales(n, seed):
    rng = np.random.default_rng(seed)
    a = (np.abs(rng.standard_normal(n)) * 0.02).astype(np.float32)
    a[:: 1031] = np.float32(7e5)          # wide exponents: the tree-ordered path
    return a


def test_noalloc_equals_workspace_entry_on_consecutive_calls():
    cases = [scales(1835008, 1),                     # the 8192 x 28672 layer's scales at block 128
             scales(70001, 2),                       # smaller: a new, shorter tree
             crafted_inputs.mean_two_level()]        # order-sensitive mean
    for i, a in enumerate(cases):
        ag = torch.from_numpy(a).cuda()
        want = call(ag, 256, noalloc=False)
        got = call(ag, 256, noalloc=True)
        for g, w, what in zip(got, want, ("codes", "group scales", "offset", "table")):
            assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), (i, what)
