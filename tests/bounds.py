"""Error bounds for the matmul parity tests (gemv_4bit, gemm_4bit and the
backward), derived from the arithmetic the kernels are allowed to do.

The oracle's reference is Y = X @ W_hat^T in float64 over the fp32 dequantized
weight W_hat.  The kernels differ from it in three ways only:

1. 16-bit activations (bf16 / fp16) multiply the weight rounded to the
   activations' type: either the rounded code value times the fp32 block
   scale, or the rounded product.  Either way each weight carries a relative
   error of at most one unit roundoff, u_w = 2^-8 for bf16 (8 significant
   bits) or 2^-11 for fp16 (11 bits).
   fp32 activations multiply the code value and the block scale in fp32,
   which differs from the once-rounded fp32 weight by at most 2^-24 relative.
2. Products are summed in fp32 in some order: with at most K + 16 roundings
   along any summation path (K products, the block scales, the cross-lane
   and cross-wave sums), the worst case is (K + 16) 2^-24 of sum |x w|.
3. A 16-bit output is rounded once more (2^-8 bf16, 2^-11 fp16).

Per element this gives the rigorous first-order bound
    |y - ref| <= (u_w + (K + 16) 2^-24) sum_k |x_k| |w_k| + u_out |ref|
(times 1.01 for second-order terms, plus the absolute error of a rounding
into the subnormal range of the weight or output type), checked on every
compared output.

Over the whole output the relative L2 error must stay within the per-dtype
tolerances ("Feat/mps gemm 4bit bf16", "Correctness": matmuls agree within
documented per-dtype tolerances): 1e-3 for fp32 operands accumulated into fp32
outputs, 2e-2 for bf16 / fp16 outputs.  With 16-bit activations and fp32
outputs the weight rounding alone makes E|dy|^2 <= u_w^2 E|y|^2 for
zero-mean random activations, so the bound is u_w + (K + 16) 2^-24:
4.2e-3 for bf16 at K = 4096, 4.8e-3 at K = 14336; 7.3e-4 for fp16 at K = 4096.
(Measured: about 1.3e-3 for bf16 with NF4 or FP4 codes, the rms of the
table values' own bf16 rounding errors.)"""
from __future__ import annotations

import numpy as np

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 2.0 ** -24}
U_OUT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 0.0}
U32 = 2.0 ** -24
# half the spacing of the subnormals: the absolute part of a rounding below
# the smallest normal number (fp16 weights or outputs under 2^-14)
ABS = {"bf16": 2.0 ** -134, "fp16": 2.0 ** -25, "fp32": 2.0 ** -150}


def _name(dt) -> str:
    s = str(dt)
    for k in ("bfloat16", "float16", "float32"):
        if s.endswith(k):
            return {"bfloat16": "bf16", "float16": "fp16", "float32": "fp32"}[k]
    return s


def rel_l2_tol(xdt, ydt, K: int) -> float:
    """Relative L2 bound over the whole output (see the module docstring)."""
    xdt, ydt = _name(xdt), _name(ydt)
    if ydt != "fp32":
        return 2e-2
    if xdt == "fp32":
        return 1e-3
    return U[xdt] + (K + 16) * U32


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def check_matmul(got, X, W, xdt, ydt, what="", bias=None):
    """got [M, N] against X [M, K] @ W [N, K]^T (+ bias [N]) in float64:
    relative L2 over all of it and the per-element bound on every element
    (the bias adds one fp32 rounding).  Returns the relative L2 error."""
    X = np.asarray(X, np.float64).reshape(-1, np.asarray(W).shape[1])
    W = np.asarray(W, np.float64)
    got = np.asarray(got, np.float64).reshape(X.shape[0], W.shape[0])
    ref = X @ W.T
    u_bias = 0.0
    if bias is not None:
        ref = ref + np.asarray(bias, np.float64).reshape(1, -1)
        u_bias = U32
    K = X.shape[1]
    xdt, ydt = _name(xdt), _name(ydt)
    err = rel_l2(got, ref)
    tol = rel_l2_tol(xdt, ydt, K)
    assert err <= tol, f"{what}: relative L2 {err:.3e} > {tol:.3e}"
    mag = np.abs(X) @ np.abs(W).T
    xsum = np.abs(X).sum(axis=1, keepdims=True)
    bound = 1.01 * ((U[xdt] + (K + 16) * U32) * mag + ABS[xdt] * xsum
                    + (U_OUT[ydt] + u_bias) * np.abs(ref) + ABS[ydt])
    bad = np.argwhere(np.abs(got - ref) > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements outside the per-element bound, first "
                           f"{bad[:4].tolist()}: got {got[tuple(bad[0])]}, want {ref[tuple(bad[0])]}, "
                           f"bound {bound[tuple(bad[0])]:.3e}")
    return err


def check_backward(got, dY, W, dydt, dxdt, what=""):
    """dX [M, K] against dY [M, N] @ W [N, K]: the same bounds with the sum
    over N (the transpose of check_matmul's contraction)."""
    W = np.asarray(W, np.float64)
    return check_matmul(got, dY, W.T, dydt, dxdt, what)
