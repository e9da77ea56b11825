"""The C ABI without a GPU: every symbol include/*.h declares is exported,
the host-side tables match the oracle bit for bit, and every precondition
comes back as its status code before anything is launched.

Pointers below are fake but well-formed host integers: validation rejects the
call before any HIP runtime call, so nothing is dereferenced."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from quantized_matvec_amd import qmv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, ALIGN, LAUNCH, HIPERR, WORKSPACE = 0, -1, -2, -3, -4, -5, -6
P = 0x7F0000010000          # 16-byte aligned fake device address
P2 = P + 0x100000
MIS = P + 4                 # misaligned
F32, F16, BF16 = 0, 1, 2
NF4, FP4 = 0, 1


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            with open(os.path.join(ROOT, "include", h)) as f:
                names |= set(re.findall(r"\b(qmv_[a-z0-9_]+)\s*\(", f.read()))
    return sorted(names)


def test_exports_every_declared_symbol(qmvlib):
    names = header_functions()
    assert len(names) == 19 and "qmv_stream_read" in names and "qmv_dynamic_code2" in names
    assert "qmv_gemm_4bit_backward_workspace" in names
    assert "qmv_double_quant_noalloc" in names
    for n in names:
        assert hasattr(qmvlib, n), n


def test_code_tables_match_oracle_bits(qmvlib):
    for qt in ("nf4", "fp4"):
        got = np.array(qmv.code_table(qt), dtype=np.float32)
        assert got.view(np.uint32).tolist() == O.code_table(qt).view(np.uint32).tolist()
    got = np.array(qmv.default_code2(), dtype=np.float32)
    assert got.view(np.uint32).tolist() == O.linear8_table().view(np.uint32).tolist()
    got = np.array(qmv.dynamic_tree_code(), dtype=np.float32)
    assert got.view(np.uint32).tolist() == O.dynamic_tree_table().view(np.uint32).tolist()


def test_status_strings(qmvlib):
    for s in (OK, INVALID, UNSUPPORTED, ALIGN, LAUNCH, HIPERR, WORKSPACE):
        assert qmvlib.qmv_status_string(s)
    assert qmvlib.qmv_status_string(12345) == b"unknown status"
    assert qmvlib.qmv_code_table(7, None) == INVALID


def _scales(absmax=0, q=0, a2=0, code2=0, off=0, bs2=256):
    return qmv._Absmax(absmax or None, q or None, a2 or None, code2 or None, off or None, bs2)


def test_quantize_preconditions(qmvlib):
    f = qmvlib.qmv_quantize_4bit
    assert f(None, F32, 64, 64, NF4, P, P2, None) == INVALID
    assert f(P, F32, 0, 64, NF4, P, P2, None) == INVALID
    assert f(P, 9, 64, 64, NF4, P, P2, None) == INVALID
    assert f(P, F32, 64, 64, 5, P, P2, None) == INVALID
    for bs in (16, 48, 8192, 0, -64):
        assert f(P, BF16, 64, bs, NF4, P, P2, None) == UNSUPPORTED
    assert f(MIS, BF16, 64, 64, NF4, P, P2, None) == ALIGN
    assert f(P, BF16, 64, 64, NF4, MIS, P2, None) == ALIGN


def test_double_quant_preconditions(qmvlib):
    f = qmvlib.qmv_double_quant
    ws = qmvlib.qmv_double_quant_workspace(1000, 256)
    assert ws == 8 * (4 + 1) + 8  # level sums (4 runs, then 1), one exponent-bound pair
    assert qmvlib.qmv_double_quant_workspace(1000, 32) == ws   # the mean's tree is fixed
    assert qmvlib.qmv_double_quant_workspace(0, 256) == 0
    assert qmvlib.qmv_double_quant_workspace(1000, 48) == 0
    assert qmvlib.qmv_dynamic_code2(None) == INVALID
    g = qmvlib.qmv_double_quant_noalloc
    assert g(P, (1 << 24) + 1, 256, None, P, P, P, P, None) == -7     # QMV_ERR_TOO_LARGE
    assert g(P, 0, 256, None, P, P, P, P, None) == INVALID
    assert g(P, 1000, 48, None, P, P, P, P, None) == UNSUPPORTED
    assert g(MIS, 1000, 256, None, P, P, P, P, None) == ALIGN
    assert qmvlib.qmv_status_string(-7)
    args = lambda **k: dict(dict(a=P, n=1000, bs2=256, code=None, q=P, a2=P, off=P, c2o=P, w=P2, wsb=ws), **k)
    call = lambda d: f(d["a"], d["n"], d["bs2"], d["code"], d["q"], d["a2"], d["off"], d["c2o"], d["w"], d["wsb"], None)
    assert call(args(n=0)) == INVALID
    assert call(args(a=0)) == INVALID
    assert call(args(bs2=100)) == UNSUPPORTED
    assert call(args(wsb=ws - 1)) == WORKSPACE
    assert call(args(w=0)) == WORKSPACE
    assert call(args(q=MIS)) == ALIGN
    bad = (ctypes.c_float * 256)(*([0.0] * 256))                # not increasing
    assert call(args(code=ctypes.cast(bad, ctypes.c_void_p))) == UNSUPPORTED
    nan = (ctypes.c_float * 256)(*[float("nan")] + list(np.linspace(0, 1, 255)))
    assert call(args(code=ctypes.cast(nan, ctypes.c_void_p))) == INVALID
    wide = np.linspace(-1, 1, 256).astype(np.float32)
    wide[0] = np.float32(-1e30)                                   # midpoint not exact
    w = (ctypes.c_float * 256)(*wide.tolist())
    assert call(args(code=ctypes.cast(w, ctypes.c_void_p))) == UNSUPPORTED
    sym = np.linspace(-1, 1, 256).astype(np.float32)              # zero midpoint (+-v)
    s = (ctypes.c_float * 256)(*sym.tolist())
    assert call(args(code=ctypes.cast(s, ctypes.c_void_p))) == UNSUPPORTED


def test_scale_descriptor_preconditions(qmvlib):
    f = qmvlib.qmv_dequantize_4bit
    ok_plain = _scales(absmax=P2)
    both = _scales(absmax=P2, q=P, a2=P, code2=P, off=P)
    neither = _scales()
    partial = _scales(q=P, a2=P)
    bad_bs2 = _scales(q=P, a2=P, code2=P, off=P, bs2=100)
    mis = _scales(q=P, a2=MIS, code2=P, off=P)
    assert f(P, None, 64, 64, NF4, P, BF16, None) == INVALID
    for sc, want in ((both, INVALID), (neither, INVALID), (partial, INVALID),
                     (bad_bs2, UNSUPPORTED), (mis, ALIGN)):
        assert f(P, ctypes.byref(sc), 64, 64, NF4, P, BF16, None) == want
    assert f(P, ctypes.byref(ok_plain), 64, 48, NF4, P, BF16, None) == UNSUPPORTED
    assert f(P, ctypes.byref(ok_plain), 64, 64, NF4, P, 3, None) == INVALID
    assert f(P, ctypes.byref(ok_plain), -1, 64, NF4, P, BF16, None) == INVALID
    assert f(MIS, ctypes.byref(ok_plain), 64, 64, NF4, P, BF16, None) == ALIGN
    g = qmvlib.qmv_dequantize_absmax
    assert g(ctypes.byref(both), 10, P, None) == INVALID
    assert g(ctypes.byref(ok_plain), 0, P, None) == INVALID


def test_matmul_preconditions(qmvlib):
    sc = _scales(absmax=P2)
    gv, gm = qmvlib.qmv_gemv_4bit, qmvlib.qmv_gemm_4bit
    r = ctypes.byref(sc)
    assert gv(P, BF16, 9, 64, 64, P, r, 64, NF4, P, BF16, None, None) == UNSUPPORTED   # M > 8
    assert gv(P, BF16, 0, 64, 64, P, r, 64, NF4, P, BF16, None, None) == INVALID
    assert gv(P, BF16, 1, 0, 64, P, r, 64, NF4, P, BF16, None, None) == INVALID
    assert gv(P, BF16, 1, 64, 96, P, r, 64, NF4, P, BF16, None, None) == UNSUPPORTED   # K % bs
    assert gv(P, BF16, 1, 64, 48, P, r, 32, NF4, P, BF16, None, None) == UNSUPPORTED   # K % 32
    assert gv(P, BF16, 1, 64, 64, P, r, 64, NF4, MIS, BF16, None, None) == ALIGN
    assert gv(None, BF16, 1, 64, 64, P, r, 64, NF4, P, BF16, None, None) == INVALID
    assert gv(P, BF16, 1, 64, 64, P, r, 64, NF4, P, BF16, P + 1, None) == ALIGN       # bias element
    assert gv(P, BF16, 1, 64, 64, P, r, 64, NF4, P, F32, P + 2, None) == ALIGN
    assert gm(P, BF16, 8, 64, 64, P, r, 100, NF4, P, BF16, None, None) == UNSUPPORTED
    assert gm(P, BF16, 8, 64, 64, P, None, 64, NF4, P, BF16, None, None) == INVALID
    assert gm(P, BF16, 8, 64, 64, P, r, 64, 2, P, BF16, None, None) == INVALID
    assert gm(P, 7, 8, 64, 64, P, r, 64, NF4, P, BF16, None, None) == INVALID
    assert gm(P, F16, 8, 64, 64, P, r, 64, NF4, P, F16, P + 1, None) == ALIGN
    gb = qmvlib.qmv_gemm_4bit_backward  # dY [M, N] @ W_hat [N, K]
    assert gb(P, F32, 8, 64, 64, P, r, 64, NF4, P, BF16, None, 0, None) == UNSUPPORTED    # dY 16-bit only
    assert gb(P, BF16, 8, 48, 64, P, r, 64, NF4, P, BF16, None, 0, None) == UNSUPPORTED   # N % 32
    assert gb(P, BF16, 8, 64, 96, P, r, 64, NF4, P, BF16, None, 0, None) == UNSUPPORTED   # K % bs
    assert gb(P, BF16, 0, 64, 64, P, r, 64, NF4, P, BF16, None, 0, None) == INVALID
    assert gb(None, BF16, 8, 64, 64, P, r, 64, NF4, P, BF16, None, 0, None) == INVALID
    assert gb(P, BF16, 8, 64, 64, P, r, 64, NF4, MIS, BF16, None, 0, None) == ALIGN
    # the split reduction's workspace: sized by its query, checked before any launch
    need = qmvlib.qmv_gemm_4bit_backward_workspace(512, 14336, 4096, 64)
    assert need > 0 and need % 256 == 0
    assert qmvlib.qmv_gemm_4bit_backward_workspace(512, 14336, 4096, 32) == 0   # blocks < 64: no split
    assert qmvlib.qmv_gemm_4bit_backward_workspace(512, 14336, 4000, 32) == 0   # K % 256
    WS = 0x100000
    assert gb(P, BF16, 512, 14336, 4096, P, r, 64, NF4, P, BF16, None, 0, None) == WORKSPACE
    assert gb(P, BF16, 512, 14336, 4096, P, r, 64, NF4, P, BF16, WS, need - 1, None) == WORKSPACE
    assert gb(P, BF16, 512, 14336, 4096, P, r, 64, NF4, P, BF16, WS + 8, need, None) == WORKSPACE


def test_binding_refuses_cpu_tensors(qmvlib):
    import torch
    with pytest.raises(ValueError):
        qmv.quantize_4bit(torch.zeros(64))


def test_blockwise_preconditions(qmvlib):
    fq, fd = qmvlib.qmv_quantize_blockwise, qmvlib.qmv_dequantize_blockwise
    assert fq(None, F32, 64, 64, None, P, P2, None) == INVALID
    assert fq(P, F32, 0, 64, None, P, P2, None) == INVALID
    assert fq(P, 9, 64, 64, None, P, P2, None) == INVALID
    for bs in (16, 48, 8192, 0):
        assert fq(P, BF16, 64, bs, None, P, P2, None) == UNSUPPORTED
        assert fd(P, P2, 64, bs, None, P, F32, None) == UNSUPPORTED
    assert fq(MIS, BF16, 64, 64, None, P, P2, None) == ALIGN
    assert fq(P, BF16, 64, 64, None, P, MIS, None) == ALIGN
    bad = (ctypes.c_float * 256)(*([0.0] * 256))                  # not increasing
    assert fq(P, BF16, 64, 64, ctypes.cast(bad, ctypes.c_void_p), P, P2, None) == UNSUPPORTED
    assert fd(P, P2, 64, 64, ctypes.cast(bad, ctypes.c_void_p), P, F32, None) == UNSUPPORTED
    assert fd(None, P2, 64, 64, None, P, F32, None) == INVALID
    assert fd(P, P2, -5, 64, None, P, F32, None) == INVALID
    assert fd(P, P2, 64, 64, None, P, 3, None) == INVALID
    assert fd(P, P2, 64, 64, None, MIS, BF16, None) == ALIGN


def test_embedding_preconditions(qmvlib):
    f = qmvlib.qmv_embedding_4bit
    sc = _scales(absmax=P2)
    r = ctypes.byref(sc)
    assert f(None, 4, 10, 64, P, r, 64, NF4, P2, BF16, None) == INVALID
    assert f(P, 0, 10, 64, P, r, 64, NF4, P2, BF16, None) == INVALID
    assert f(P, 4, 0, 64, P, r, 64, NF4, P2, BF16, None) == INVALID
    assert f(P, 4, 10, 0, P, r, 64, NF4, P2, BF16, None) == INVALID
    assert f(P, 4, 1 << 40, 1 << 30, P, r, 64, NF4, P2, BF16, None) == INVALID   # V * D overflows
    assert f(P, 4, 10, 64, P, r, 48, NF4, P2, BF16, None) == UNSUPPORTED
    assert f(P, 4, 10, 64, P, r, 64, 3, P2, BF16, None) == INVALID
    assert f(P, 4, 10, 64, P, None, 64, NF4, P2, BF16, None) == INVALID
    assert f(P + 4, 4, 10, 64, P, r, 64, NF4, P2, BF16, None) == ALIGN
    assert f(P, 4, 10, 64, P, r, 64, NF4, MIS, BF16, None) == ALIGN


def test_stream_read_preconditions(qmvlib):
    f = qmvlib.qmv_stream_read
    assert f(None, 1024, P2, None) == INVALID
    assert f(P, 1024, None, None) == INVALID
    assert f(P, 0, P2, None) == INVALID
    assert f(P, 1000, P2, None) == INVALID          # not a multiple of 16
    assert f(P + 8, 1024, P2, None) == ALIGN
    assert f(P, 1024, P2 + 2, None) == ALIGN


# ---------------------------------------------------------------- Python-side refusals
def _state(N=64, K=128, bs=64, dq=False, nb=None, packed_bytes=None):
    import torch
    nb = (N * K) // bs if nb is None else nb
    packed = torch.zeros((N * K) // 2 if packed_bytes is None else packed_bytes, dtype=torch.uint8)
    if dq:
        st = qmv.QuantState((N, K), torch.bfloat16, bs, "nf4", None,
                            torch.zeros(nb, dtype=torch.uint8), torch.zeros(-(-nb // 256)),
                            torch.zeros(1), torch.zeros(256), 256)
    else:
        st = qmv.QuantState((N, K), torch.bfloat16, bs, "nf4", absmax=torch.zeros(nb))
    return packed, st


@pytest.mark.parametrize("dq", [False, True])
def test_binding_refuses_mismatched_state(dq):
    """Sizes that would make a kernel read past a buffer are refused in
    Python, before any device call (CPU tensors: the size checks come first)."""
    import torch
    x = torch.zeros(1, 128, dtype=torch.bfloat16)
    packed, st = _state(dq=dq, packed_bytes=100)
    with pytest.raises(ValueError, match="packed must hold"):
        qmv.gemv_4bit(x, packed, st)
    packed, st = _state(dq=dq, nb=100)
    with pytest.raises(ValueError, match="absmax"):
        qmv.gemm_4bit(x, packed, st)
    with pytest.raises(ValueError, match="absmax"):
        qmv.dequantize_4bit(packed, st)
    packed, st = _state(dq=dq)
    with pytest.raises(ValueError, match="last dimension"):
        qmv.gemv_4bit(torch.zeros(1, 127, dtype=torch.bfloat16), packed, st)
    with pytest.raises(ValueError, match="last dimension"):
        qmv.gemm_4bit_backward(torch.zeros(2, 63, dtype=torch.bfloat16), packed, st)
    if dq:
        st.code2 = torch.zeros(255)
        with pytest.raises(ValueError, match="code2"):
            qmv.gemv_4bit(x, packed, st)
        st.code2 = torch.zeros(256)
        st.absmax = torch.zeros(st.nblocks)
        with pytest.raises(ValueError, match="not both"):
            qmv.gemv_4bit(x, packed, st)
    # a well-formed state on the CPU gets as far as the device check
    packed, st = _state(dq=dq)
    with pytest.raises(ValueError, match="GPU tensor"):
        qmv.gemv_4bit(x, packed, st)


# ---------------------------------------------------------------- gemm launch extents
@pytest.mark.parametrize("M", [65, 200, 447, 448, 512, 1000, 1024, 2048, 4096, 4096 + 77])
@pytest.mark.parametrize("N", [14336, 1000, 28672])
def test_gemm_tiles_cover_the_output_once_within_bounds(qmvlib, M, N):
    """The workgroup tiles of gemm_4bit's launch (from the launcher's own
    choice and tile mapping): every one lies inside [0, M) x [0, N), so no
    workgroup reads a row of A past M * K or writes C past M * N, and
    together they cover every output exactly once."""
    K = 4096
    kind = ctypes.c_int32(-1)
    n = qmvlib.qmv_gemm_4bit_plan(M, N, K, 64, None, 0, ctypes.byref(kind))
    assert n > 0
    tiles = (ctypes.c_int64 * (4 * n))()
    assert qmvlib.qmv_gemm_4bit_plan(M, N, K, 64, tiles, n, ctypes.byref(kind)) == n
    assert kind.value == (3 if M >= 448 else 2)
    t = np.array(tiles, dtype=np.int64).reshape(n, 4)
    r0, c0, nr, nc = t.T
    assert (r0 >= 0).all() and (c0 >= 0).all() and (nr > 0).all() and (nc > 0).all()
    assert (r0 + nr <= M).all() and (c0 + nc <= N).all()          # A rows < M, C elements < M * N
    assert int((nr * nc).sum()) == M * N                           # no overlap, given full cover below
    cover = np.zeros((M, N), dtype=np.uint8)
    for a, b, c, d in t:
        cover[a:a + c, b:b + d] += 1
    assert cover.min() == 1 and cover.max() == 1


def test_gemm_plan_refuses_bad_shapes(qmvlib):
    kind = ctypes.c_int32(-1)
    assert qmvlib.qmv_gemm_4bit_plan(0, 10, 64, 64, None, 0, ctypes.byref(kind)) == INVALID
    assert qmvlib.qmv_gemm_4bit_plan(10, 10, 96, 64, None, 0, ctypes.byref(kind)) == UNSUPPORTED
    assert qmvlib.qmv_gemm_4bit_plan(10, 10, 64, 64, None, 0, None) == INVALID
