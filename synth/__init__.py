"""Seeded synthetic inputs for the W4A16 / W4A8 linear layer.

This module only draws random numbers and shapes.  It holds none of the
method's arithmetic (no quantization, packing, dequantization or matmul), so
both the CPU oracle and the GPU path may take their inputs from it.

Recipe (the same for every workload; one ``torch.Generator('cpu')`` per call,
seeded, draws taken in this fixed order):

1. ``W`` fp32 ~ N(0, 0.02) of shape [N, K] (out, in).
2. Optional outlier input channels: ``round(0.01 * K)`` column indices from a
   seeded permutation of ``range(K)``; those columns are multiplied by 10
   (salient input channels, the kind activation-aware quantization protects).
   ``W`` is then rounded to fp16 once.
3. ``X`` fp32 ~ N(0, 1) of shape [M, K]; optionally every token row is scaled
   by ``0.5 + 3.5 * U(0, 1)`` (per-token RMS spread of 0.5x..4x, the
   prefill-shaped workload); then rounded to fp16.
4. Optional RMSNorm weight ``gamma`` fp16 ~ 1 + 0.1 * N(0, 1) of shape [K].

Because ``W`` is drawn first, the same (seed, N, K, outliers) gives the same
weight for every M.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

# Llama-2-13B projection shapes (K = in_features, N = out_features):
# fused QKV, attention output, fused gate+up, MLP down.
LLAMA2_13B = {
    "qkv": (5120, 15360),
    "o": (5120, 5120),
    "gate_up": (5120, 27648),
    "down": (13824, 5120),
}


@dataclass
class LinearInputs:
    w: torch.Tensor            # fp16 [N, K]
    x: torch.Tensor            # fp16 [M, K]
    gamma: torch.Tensor | None  # fp16 [K] or None
    outlier_cols: torch.Tensor | None  # int64 indices into K, or None


def make_linear(M: int, N: int, K: int, seed: int = 0, outliers: bool = False,
                rms_spread: bool = False, with_gamma: bool = False) -> LinearInputs:
    """Draw (W, X[, gamma]) for one linear layer following the module recipe."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    w = torch.randn(N, K, generator=g, dtype=torch.float32) * 0.02
    cols = None
    if outliers:
        n_out = int(round(0.01 * K))
        cols = torch.randperm(K, generator=g)[:n_out]
        w[:, cols] *= 10.0
    w16 = w.to(torch.float16)
    del w
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    if rms_spread and M > 0:
        r = 0.5 + 3.5 * torch.rand(M, 1, generator=g, dtype=torch.float32)
        x = x * r
    x16 = x.to(torch.float16)
    gamma = None
    if with_gamma:
        gamma = (1.0 + 0.1 * torch.randn(K, generator=g, dtype=torch.float32)).to(torch.float16)
    return LinearInputs(w=w16, x=x16, gamma=gamma, outlier_cols=cols)


def make_activations(M: int, K: int, seed: int = 1, rms_spread: bool = False) -> torch.Tensor:
    """fp16 [M, K] activations alone (X ~ N(0,1), optional per-token RMS spread)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    if rms_spread and M > 0:
        x = x * (0.5 + 3.5 * torch.rand(M, 1, generator=g, dtype=torch.float32))
    return x.to(torch.float16)


def uniform_ints(shape, lo: int, hi: int, seed: int) -> torch.Tensor:
    """int64 tensor of uniform integers in [lo, hi] (inclusive)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, dtype=torch.int64)


def normal(shape, std: float, seed: int) -> torch.Tensor:
    """fp32 tensor ~ N(0, std^2)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32) * std


# The five workloads, as (name, list of (M, N, K, kwargs)).
def workloads():
    """All parity/bench cases keyed by workload name."""
    out = {}
    out["single_m8_4096"] = [(8, 4096, 4096, dict(outliers=False))]
    out["decode_13b"] = [(m, n, k, dict(outliers=True))
                         for (k, n) in LLAMA2_13B.values() for m in (1, 4, 16)]
    out["crossover_5120x13824"] = [(m, 13824, 5120, dict(outliers=True))
                                   for m in (1, 2, 8, 16, 32, 64, 128, 256)]
    out["prefill_13b"] = [(4096, n, k, dict(outliers=True, rms_spread=True))
                          for (k, n) in ((5120, 27648), (5120, 5120), (13824, 5120))]
    out["w4a8_5120x13824"] = [(m, 13824, 5120, dict(outliers=True, rms_spread=True, with_gamma=True))
                              for m in (1, 16, 256, 4096)]
    return out
