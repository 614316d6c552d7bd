"""Helpers for the GPU parity tests (acceptance metric, sampling, device)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

# Acceptance for fp16 outputs: |Y_gpu - Y_ref| / (||x_m|| * ||w_n||) <= 2e-3 per output,
# where w_n is row n of the dequantized weight.  Worst-case budget with fp32
# accumulation: fp16 output rounding 2^-11 + fp32 sums K * 2^-24 (8.2e-4 at K = 13824)
# + fp16 rounding of each dequantized weight 2^-11 (Cauchy-Schwarz) = 1.8e-3.
TOL = 2e-3


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def normalized_error(y_gpu, y_ref, xnorm, wnorm):
    """Max over outputs of |y_gpu - y_ref| / (||x_m|| ||w_n||); outputs with a zero
    denominator must be exactly zero (returned as +inf otherwise)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.outer(np.asarray(xnorm, np.float64), np.asarray(wnorm, np.float64))
    diff = np.abs(y_gpu - y_ref)
    zero = den == 0
    if np.any(zero & (y_gpu != 0)):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(zero, 0.0, diff / np.where(zero, 1.0, den))
    return float(e.max()) if e.size else 0.0


def sample_idx(n: int, k: int, seed: int, must=()):
    """Sorted sample of k indices in [0, n) that always includes the ends and `must`."""
    rng = np.random.default_rng(seed)
    base = {0, n - 1, *[m for m in must if 0 <= m < n]}
    extra = rng.choice(n, size=min(n, k), replace=False)
    return np.array(sorted(base | set(int(v) for v in extra)), dtype=np.int64)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
