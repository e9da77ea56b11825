"""Seeded synthetic inputs shaped like LLM linear layers.

This module only draws random numbers and rounds them into their storage
dtype with torch's own CPU conversions (float64 -> fp32 -> bf16, each round to
nearest even).  It holds none of the codec's arithmetic, so the GPU path and
the CPU oracle can both be fed from it.

Recipe: ``numpy.random.default_rng(100 * cfg + role)``; ``standard_normal`` in
float64 times sigma; outliers are ``rng.choice(numel, round(frac * numel),
replace=False)`` positions (their own seed) multiplied by 20 in float64 before
rounding.  Roles: 0 first weight, 1 second weight, 2 activations of the first
weight, 3 outlier positions of the first weight, 4 outlier positions of the
second weight, 5 activations of the second weight.

The workloads follow the shapes of 8B-class (4096 / 14336) and 70B-class
(8192 / 28672) dense MLP layers; weights are Gaussian because NF4 is built for
normally distributed weights ("mps-bitsandbytes 0.4.7", section "Features").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["gaussian", "Workload", "WORKLOADS", "weight", "activations"]

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def gaussian(shape, sigma: float, seed: int, dtype: str = "bf16",
             outlier_frac: float = 0.0, outlier_seed: int | None = None,
             outlier_scale: float = 20.0) -> torch.Tensor:
    """CPU tensor of N(0, sigma^2) draws in ``dtype`` ("fp32", "bf16", "fp16")."""
    n = int(np.prod(shape))
    v = np.random.default_rng(seed).standard_normal(n) * sigma
    if outlier_frac > 0.0:
        k = int(round(outlier_frac * n))
        idx = np.random.default_rng(outlier_seed).choice(n, k, replace=False)
        v[idx] *= outlier_scale
    t = torch.from_numpy(v.reshape(shape)).to(torch.float32)
    return t if dtype == "fp32" else t.to(_DT[dtype])


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity configuration."""
    cfg: int
    name: str
    weights: tuple            # ((N, K), ...) one entry per weight matrix
    sigma: float
    w_dtype: str
    blocksize: int
    quant_types: tuple
    double_quant: bool
    outlier_frac: float
    x_dtype: str
    y_dtype: str
    ms: tuple                 # activation row counts exercised
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload(1, "nf4 round trip + gemv, fp32 1024x1024", ((1024, 1024),), 0.02,
                "fp32", 64, ("nf4",), False, 0.0, "fp32", "fp32", (1,)),
    2: Workload(2, "gemv decode + codec throughput, bf16 4096x4096", ((4096, 4096),), 0.02,
                "bf16", 64, ("nf4",), False, 0.0, "bf16", "bf16", (1,)),
    3: Workload(3, "LLM MLP up/down, outliers, double-quant absmax", ((14336, 4096), (4096, 14336)),
                0.02, "bf16", 64, ("nf4", "fp4"), True, 0.001, "bf16", "bf16", (1,)),
    4: Workload(4, "gemm prefill 14336x4096", ((14336, 4096),), 0.02,
                "bf16", 64, ("nf4",), False, 0.0, "bf16", "bf16", (8, 32, 128, 512)),
    5: Workload(5, "large-layer sweep 8192x28672 / 28672x8192, double-quant", ((8192, 28672), (28672, 8192)),
                0.015, "bf16", 128, ("nf4", "fp4"), True, 0.0, "bf16", "bf16", (1, 2, 4, 8)),
}


def weight(cfg: int, which: int = 0) -> torch.Tensor:
    """Weight ``which`` (0 or 1) of workload ``cfg`` as a CPU tensor [N, K]."""
    w = WORKLOADS[cfg]
    shape = w.weights[which]
    return gaussian(shape, w.sigma, 100 * cfg + which, w.w_dtype,
                    w.outlier_frac, 100 * cfg + 3 + which)


def activations(cfg: int, which: int = 0, m: int | None = None) -> torch.Tensor:
    """Activations [M, K] for weight ``which`` of workload ``cfg``; rows beyond
    the first M of the largest M are never drawn differently (prefix-stable)."""
    w = WORKLOADS[cfg]
    K = w.weights[which][1]
    mmax = max(w.ms)
    x = gaussian((mmax, K), 1.0, 100 * cfg + (2 if which == 0 else 5), w.x_dtype)
    return x[: (mmax if m is None else m)].contiguous()
