"""Python binding of libqmv.so (ctypes).

Argument marshalling only: torch supplies device memory and the current HIP
stream, and every step of every operation runs in the library's HIP kernels.
There is no CPU or PyTorch fallback; if the library is not built, or a call's
arguments are refused, these functions raise.

Names follow the op set of the pages ("Feat/mps gemm 4bit bf16", table "What
runs natively now"; "mps-bitsandbytes 0.4.7", section "Functional API").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "QmvError", "QuantState", "lib", "library_path", "quantize_4bit", "double_quant",
    "dequantize_absmax", "dequantize_4bit", "gemv_4bit", "gemm_4bit", "code_table",
    "default_code2", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libqmv.so")

STATUS = {0: "QMV_OK", -1: "QMV_ERR_INVALID_ARG", -2: "QMV_ERR_UNSUPPORTED",
          -3: "QMV_ERR_ALIGNMENT", -4: "QMV_ERR_LAUNCH", -5: "QMV_ERR_HIP",
          -6: "QMV_ERR_WORKSPACE", -7: "QMV_ERR_TOO_LARGE"}
_QT = {"nf4": 0, "fp4": 1}
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class QmvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_string(status)})")


class _Absmax(ctypes.Structure):
    _fields_ = [("absmax", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax2", ctypes.c_void_p), ("code2", ctypes.c_void_p),
                ("offset", ctypes.c_void_p), ("blocksize2", ctypes.c_int32)]


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(library_path):
        raise ImportError(f"{library_path} is missing: build it with "
                          "`python -m quantized_matvec_amd.build`")
    L = ctypes.CDLL(library_path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    ap = ctypes.POINTER(_Absmax)
    sig = {
        "qmv_quantize_4bit": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, ctypes.c_int, vp, vp, vp]),
        "qmv_double_quant_workspace": (sz, [i64, i32]),
        "qmv_double_quant": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "qmv_double_quant_noalloc": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, vp, vp, vp]),
        "qmv_dequantize_absmax": (ctypes.c_int, [ap, i64, vp, vp]),
        "qmv_dequantize_4bit": (ctypes.c_int, [vp, ap, i64, i32, ctypes.c_int, vp, ctypes.c_int, vp]),
        "qmv_gemv_4bit": (ctypes.c_int, [vp, ctypes.c_int, i32, i64, i64, vp, ap, i32,
                                         ctypes.c_int, vp, ctypes.c_int, vp, vp]),
        "qmv_gemm_4bit": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, i64, vp, ap, i32,
                                         ctypes.c_int, vp, ctypes.c_int, vp, vp]),
        "qmv_quantize_blockwise": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, vp, vp, vp, vp]),
        "qmv_dequantize_blockwise": (ctypes.c_int, [vp, vp, i64, i32, vp, vp, ctypes.c_int, vp]),
        "qmv_gemm_4bit_backward": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, i64, vp, ap, i32,
                                                  ctypes.c_int, vp, ctypes.c_int, vp, sz, vp]),
        "qmv_gemm_4bit_backward_workspace": (sz, [i64, i64, i64, i32]),
        "qmv_embedding_4bit": (ctypes.c_int, [vp, i64, i64, i64, vp, ap, i32, ctypes.c_int, vp,
                                              ctypes.c_int, vp]),
        "qmv_stream_read": (ctypes.c_int, [vp, i64, vp, vp]),
        "qmv_gemm_4bit_plan": (i64, [i64, i64, i64, i32, vp, i64, vp]),
        "qmv_code_table": (ctypes.c_int, [ctypes.c_int, vp]),
        "qmv_default_code2": (ctypes.c_int, [vp]),
        "qmv_dynamic_code2": (ctypes.c_int, [vp]),
        "qmv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _LIB = L
    return L


def _status_string(status: int) -> str:
    try:
        return lib().qmv_status_string(status).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise QmvError(rc, what)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    """Contiguous, 16-byte aligned device tensor (clones views that are not)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous() or t.data_ptr() % 16:
        t = t.contiguous().clone()
    return t


@dataclass
class QuantState:
    """Everything dequantize / gemv / gemm need besides the packed codes."""
    shape: tuple
    dtype: torch.dtype
    blocksize: int
    quant_type: str
    absmax: Optional[torch.Tensor] = None        # plain fp32 scales
    absmax_q: Optional[torch.Tensor] = None      # double-quantized scales
    absmax2: Optional[torch.Tensor] = None
    offset: Optional[torch.Tensor] = None
    code2: Optional[torch.Tensor] = None
    blocksize2: int = 256

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n

    @property
    def nblocks(self) -> int:
        return -(-self.numel // self.blocksize)

    @property
    def double_quant(self) -> bool:
        return self.absmax is None

    def _c(self) -> _Absmax:
        if self.absmax is not None:
            return _Absmax(self.absmax.data_ptr(), None, None, None, None, 0)
        return _Absmax(None, self.absmax_q.data_ptr(), self.absmax2.data_ptr(),
                       self.code2.data_ptr(), self.offset.data_ptr(), self.blocksize2)


def quantize_4bit(W: torch.Tensor, blocksize: int = 64, quant_type: str = "nf4",
                  double_quant: bool = False, blocksize2: int = 256,
                  code2: Optional[list] = None):
    """Returns (packed uint8 [ceil(numel/2)], QuantState)."""
    W = _dev(W, "W")
    numel = W.numel()
    packed = torch.empty((numel + 1) // 2, dtype=torch.uint8, device=W.device)
    absmax = torch.empty(-(-numel // blocksize), dtype=torch.float32, device=W.device)
    _check(lib().qmv_quantize_4bit(W.data_ptr(), _DT[W.dtype], numel, blocksize, _QT[quant_type],
                                   packed.data_ptr(), absmax.data_ptr(), _stream(W)),
           "quantize_4bit")
    state = QuantState(tuple(W.shape), W.dtype, blocksize, quant_type, absmax=absmax)
    if double_quant:
        q, a2, off, c2 = _double_quant(absmax, blocksize2, code2)
        state = QuantState(tuple(W.shape), W.dtype, blocksize, quant_type, None, q, a2, off, c2,
                           blocksize2)
    return packed, state


def _double_quant(absmax: torch.Tensor, blocksize2: int = 256, code2: Optional[list] = None):
    """Returns (absmax_q uint8, absmax2 fp32, offset fp32 [1], code2 fp32 [256])."""
    absmax = _dev(absmax, "absmax")
    n = absmax.numel()
    dev = absmax.device
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    a2 = torch.empty(-(-n // blocksize2), dtype=torch.float32, device=dev)
    off = torch.empty(1, dtype=torch.float32, device=dev)
    c2 = torch.empty(256, dtype=torch.float32, device=dev)
    wsb = lib().qmv_double_quant_workspace(n, blocksize2)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    host = None
    if code2 is not None:
        host = (ctypes.c_float * 256)(*[float(v) for v in code2])
    _check(lib().qmv_double_quant(absmax.data_ptr(), n, blocksize2,
                                  ctypes.cast(host, ctypes.c_void_p) if host is not None else None,
                                  q.data_ptr(), a2.data_ptr(), off.data_ptr(), c2.data_ptr(),
                                  ws.data_ptr(), ws.numel(), _stream(absmax)), "double_quant")
    return q, a2, off, c2


double_quant = _double_quant


def dequantize_absmax(state: QuantState) -> torch.Tensor:
    ref = state.absmax if state.absmax is not None else state.absmax_q
    out = torch.empty(state.nblocks, dtype=torch.float32, device=ref.device)
    c = state._c()
    _check(lib().qmv_dequantize_absmax(ctypes.byref(c), state.nblocks, out.data_ptr(),
                                       _stream(ref)), "dequantize_absmax")
    return out


def dequantize_4bit(packed: torch.Tensor, state: QuantState, out: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    _check_state(packed, state)
    packed = _dev(packed, "packed")
    if out is None:
        out = torch.empty(state.shape, dtype=out_dtype or state.dtype, device=packed.device)
    elif not out.is_contiguous() or out.numel() != state.numel or out.data_ptr() % 16:
        raise ValueError("out must be contiguous, 16-byte aligned and hold numel elements")
    c = state._c()
    _check(lib().qmv_dequantize_4bit(packed.data_ptr(), ctypes.byref(c), state.numel,
                                     state.blocksize, _QT[state.quant_type], out.data_ptr(),
                                     _DT[out.dtype], _stream(packed)), "dequantize_4bit")
    return out


def _check_state(packed: torch.Tensor, state: QuantState, device=None) -> None:
    """Refuses a packed tensor or QuantState whose sizes or devices do not
    match, before anything reaches a kernel (which would otherwise read past
    the ends of the buffers)."""
    if packed.dtype != torch.uint8 or packed.numel() != (state.numel + 1) // 2:
        raise ValueError(f"packed must hold ceil(numel / 2) = {(state.numel + 1) // 2} uint8 "
                         f"bytes, got {packed.numel()} of {packed.dtype}")
    nb = state.nblocks
    if state.absmax is not None:
        parts = {"absmax": (state.absmax, nb, torch.float32)}
        if any(t is not None for t in (state.absmax_q, state.absmax2, state.offset, state.code2)):
            raise ValueError("a QuantState has either plain or double-quantized scales, not both")
    else:
        if any(t is None for t in (state.absmax_q, state.absmax2, state.offset, state.code2)):
            raise ValueError("double-quantized scales need absmax_q, absmax2, offset and code2")
        parts = {"absmax_q": (state.absmax_q, nb, torch.uint8),
                 "absmax2": (state.absmax2, -(-nb // state.blocksize2), torch.float32),
                 "offset": (state.offset, 1, torch.float32),
                 "code2": (state.code2, 256, torch.float32)}
    dev = packed.device if device is None else device
    for name, (t, n, dt) in parts.items():
        if t.numel() != n or t.dtype != dt:
            raise ValueError(f"{name} must hold {n} values of {dt}, got {t.numel()} of {t.dtype}")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the operands on {dev}")
    if packed.device != dev:
        raise ValueError(f"packed is on {packed.device}, the operands on {dev}")


def _matmul(name, x, packed, state, out, out_dtype, bias):
    if len(state.shape) != 2:
        raise ValueError("the quantized weight must be 2-D [N, K]")
    N, K = state.shape
    if x.dim() < 1 or x.shape[-1] != K:
        raise ValueError(f"x must have K = {K} elements in its last dimension, got {tuple(x.shape)}")
    _check_state(packed, state, x.device)
    packed = _dev(packed, "packed")
    x = _dev(x, "x")
    x2 = x.reshape(-1, K)
    M = x2.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or x.dtype, device=x.device)
    elif not out.is_contiguous() or out.numel() != M * N or out.data_ptr() % 16:
        raise ValueError("out must be contiguous, 16-byte aligned and hold M * N elements")
    bias_ptr = None
    if bias is not None:
        bias = _dev(bias, "bias")
        if bias.dtype != out.dtype or bias.numel() != N:
            raise ValueError("bias must hold N elements of the output dtype")
        bias_ptr = bias.data_ptr()
    c = state._c()
    f = getattr(lib(), "qmv_" + name)
    _check(f(x2.data_ptr(), _DT[x2.dtype], M, N, K, packed.data_ptr(), ctypes.byref(c),
             state.blocksize, _QT[state.quant_type], out.data_ptr(), _DT[out.dtype], bias_ptr,
             _stream(x2)), name)
    return out


def gemv_4bit(x: torch.Tensor, packed: torch.Tensor, state: QuantState,
              out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
              bias: Optional[torch.Tensor] = None):
    """y [M, N] = x [M, K] @ W_hat^T (+ bias [N]) for 1 <= M <= 8."""
    return _matmul("gemv_4bit", x, packed, state, out, out_dtype, bias)


def gemm_4bit(A: torch.Tensor, packed: torch.Tensor, state: QuantState,
              out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
              bias: Optional[torch.Tensor] = None):
    """C [M, N] = A [M, K] @ W_hat^T (+ bias [N]); A in bf16, fp16 or fp32."""
    return _matmul("gemm_4bit", A, packed, state, out, out_dtype, bias)


def _code8(code):
    if code is None:
        return None, None
    buf = (ctypes.c_float * 256)(*[float(v) for v in code])
    return ctypes.cast(buf, ctypes.c_void_p), buf


def quantize_blockwise(A: torch.Tensor, blocksize: int = 4096, code: Optional[list] = None):
    """8-bit blockwise codec: (q uint8 [numel], absmax fp32 [ceil(numel / blocksize)])."""
    A = _dev(A, "A")
    n = A.numel()
    q = torch.empty(n, dtype=torch.uint8, device=A.device)
    absmax = torch.empty(-(-n // blocksize), dtype=torch.float32, device=A.device)
    cp, _keep = _code8(code)
    _check(lib().qmv_quantize_blockwise(A.data_ptr(), _DT[A.dtype], n, blocksize, cp, q.data_ptr(),
                                        absmax.data_ptr(), _stream(A)), "quantize_blockwise")
    return q, absmax


def dequantize_blockwise(q: torch.Tensor, absmax: torch.Tensor, blocksize: int = 4096,
                         code: Optional[list] = None, out_dtype: torch.dtype = torch.float32,
                         out: Optional[torch.Tensor] = None):
    """out [numel] = code[q] * absmax[block], rounded to out_dtype."""
    q = _dev(q, "q")
    absmax = _dev(absmax, "absmax")
    n = q.numel()
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=q.device)
    elif not out.is_contiguous() or out.numel() != n or out.data_ptr() % 16:
        raise ValueError("out must be contiguous, 16-byte aligned and hold numel elements")
    cp, _keep = _code8(code)
    _check(lib().qmv_dequantize_blockwise(q.data_ptr(), absmax.data_ptr(), n, blocksize, cp,
                                          out.data_ptr(), _DT[out.dtype], _stream(q)),
           "dequantize_blockwise")
    return out


def dynamic_tree_code() -> list:
    """The library's signed dynamic-tree 8-bit table (qmv_dynamic_code2):
    256 ascending fp32 values, a decimal exponent e = 0 .. 6 taken by a run of
    leading zero bits, then 6 - e bits of linear fraction in [0.1, 1]."""
    buf = (ctypes.c_float * 256)()
    _check(lib().qmv_dynamic_code2(ctypes.cast(buf, ctypes.c_void_p)), "dynamic_code2")
    return list(buf)


_BWD_WS: dict = {}


def _backward_workspace(nbytes: int, device: torch.device) -> Optional[torch.Tensor]:
    """The backward's workspace for the current stream of ``device`` (calls in
    order on one stream can share it; a larger request replaces it)."""
    if nbytes == 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _BWD_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _BWD_WS[key] = ws
    return ws


def gemm_4bit_backward(dY: torch.Tensor, packed: torch.Tensor, state: QuantState,
                       out: Optional[torch.Tensor] = None,
                       out_dtype: Optional[torch.dtype] = None):
    """dX [M, K] = dY [M, N] @ W_hat (dY in bf16 or fp16): the input gradient of y = x @ W_hat^T."""
    if len(state.shape) != 2:
        raise ValueError("the quantized weight must be 2-D [N, K]")
    N, K = state.shape
    if dY.dim() < 1 or dY.shape[-1] != N:
        raise ValueError(f"dY must have N = {N} elements in its last dimension, got {tuple(dY.shape)}")
    _check_state(packed, state, dY.device)
    packed = _dev(packed, "packed")
    dY = _dev(dY, "dY")
    g2 = dY.reshape(-1, N)
    M = g2.shape[0]
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype or dY.dtype, device=dY.device)
    elif not out.is_contiguous() or out.numel() != M * K or out.data_ptr() % 16:
        raise ValueError("out must be contiguous, 16-byte aligned and hold M * K elements")
    ws = _backward_workspace(lib().qmv_gemm_4bit_backward_workspace(M, N, K, state.blocksize), dY.device)
    c = state._c()
    _check(lib().qmv_gemm_4bit_backward(g2.data_ptr(), _DT[g2.dtype], M, N, K, packed.data_ptr(),
                                        ctypes.byref(c), state.blocksize, _QT[state.quant_type],
                                        out.data_ptr(), _DT[out.dtype],
                                        ws.data_ptr() if ws is not None else None,
                                        ws.numel() if ws is not None else 0, _stream(g2)),
           "gemm_4bit_backward")
    return out


def embedding_4bit(idx: torch.Tensor, packed: torch.Tensor, state: QuantState,
                   out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None):
    """Rows idx of the 4-bit quantized [V, D] table: out [*idx.shape, D];
    an index outside [0, V) gives a row of zeros."""
    if len(state.shape) != 2:
        raise ValueError("the quantized table must be 2-D [V, D]")
    V, D = state.shape
    _check_state(packed, state, idx.device)
    packed = _dev(packed, "packed")
    idx = _dev(idx, "idx")
    if idx.dtype in (torch.int32, torch.int16, torch.uint8):
        idx = idx.to(torch.int64)
    if idx.dtype != torch.int64:
        raise ValueError("idx must be an integer tensor")
    T = idx.numel()
    shape = tuple(idx.shape) + (D,)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype or state.dtype, device=idx.device)
    elif not out.is_contiguous() or out.numel() != T * D or out.data_ptr() % 16:
        raise ValueError("out must be contiguous, 16-byte aligned and hold T * D elements")
    if T == 0:
        return out
    c = state._c()
    _check(lib().qmv_embedding_4bit(idx.data_ptr(), T, V, D, packed.data_ptr(), ctypes.byref(c),
                                    state.blocksize, _QT[state.quant_type], out.data_ptr(),
                                    _DT[out.dtype], _stream(idx)), "embedding_4bit")
    return out


def code_table(quant_type: str = "nf4") -> list:
    buf = (ctypes.c_float * 16)()
    _check(lib().qmv_code_table(_QT[quant_type], ctypes.cast(buf, ctypes.c_void_p)), "code_table")
    return list(buf)


def default_code2() -> list:
    buf = (ctypes.c_float * 256)()
    _check(lib().qmv_default_code2(ctypes.cast(buf, ctypes.c_void_p)), "default_code2")
    return list(buf)


def stream_read(buf: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement probe (qmv_stream_read): reads every byte of the contiguous
    device tensor `buf` once with 128-bit loads; workgroup b XORs the 32-bit
    words it read into sink[b] (sink: 8192 int32 on the device, zeroed here
    when not given; the XOR of all of it is the XOR of buf's words).
    Returns the sink; nothing synchronizes."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("stream_read: buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(8192, dtype=torch.int32, device=buf.device)
    if sink.numel() < 8192 or sink.dtype != torch.int32 or not sink.is_cuda:
        raise ValueError("stream_read: sink must be 8192 int32 on the device")
    _check(lib().qmv_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(buf)),
           "stream_read")
    return sink
