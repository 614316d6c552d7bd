"""GPU: order-independent bit-exact W4A16 GEMMs at the full Llama-2-13B shapes, through
the plan the dispatcher picks at every M of the decode, crossover and prefill workloads.

Constructed so that the exact result is reached by any summation order: integer X in
[-4, 4], random 4-bit codes and zero points (every group holds a 0 and a 15 code), and
every scale 2^-3.  Each product x (q - z) / 8 and every partial sum is a multiple of 1/8
below 2^17 in magnitude (K <= 13824, |x (q - z)| <= 60), hence exact in fp32 -- in the
skinny kernels' per-group form s (T - P - z S) too, whose T, P, S are integers below
2^20 -- so Y must equal fp16_RNE of the exact product bit for bit, whatever the split-K
or MFMA order.  One wrong code, scale or zero point anywhere in a sampled output's row
changes it.  Row 0 of X is all zeros and must give exactly 0.

The packed weights are built on the GPU from plain codes (w4_pack_codes, then
awq_import_plain, both bit-exact against the oracle in their own tests); the expected
values are plain integer arithmetic on the host (fp64 BLAS on integers: exact).
"""
import numpy as np
import pytest
import torch

import synth
import w4a16_gemm_amd as w4
from gpu_util import announce, device, sample_idx, to_np

pytestmark = pytest.mark.gpu

SHAPES = {name: kn for name, kn in synth.LLAMA2_13B.items()}  # name -> (K, N)
MS = (1, 2, 3, 4, 8, 16, 32, 64, 128, 256, 4096)

_CACHE = {}


def _weights(name, dev):
    """Codes q [N, K], zero points z [N, K/128] (host) and the packed GPU tensors."""
    if name not in _CACHE:
        _CACHE.clear()
        K, N = SHAPES[name]
        rng = np.random.default_rng(K + N)
        q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        q[:, 5::128] = 0
        q[:, 77::128] = 15
        z = rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
        words = w4.w4_pack_codes(torch.from_numpy(q).to(dev))
        zw = w4.w4_pack_codes(torch.from_numpy(z).to(dev))
        s = torch.full((N, K // 128), 0.125, dtype=torch.float16, device=dev)
        packed = w4.awq_import_plain(words, s, zw, 128, "rows")
        torch.cuda.synchronize()
        del words, zw, s
        _CACHE[name] = (q, z, packed)
    return _CACHE[name]


@pytest.mark.parametrize("M", MS)
@pytest.mark.parametrize("name", list(SHAPES))
def test_constructed_exact_full_shape(name, M):
    dev = device()
    K, N = SHAPES[name]
    announce(f"exact full {name} M={M} N={N} K={K} ws={w4.awq_gemm_workspace_bytes(M, N, K)}")
    q, z, (qw, sc, qz) = _weights(name, dev)
    rng = np.random.default_rng(M * 31 + K)
    x = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    x[0] = 0
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    w4.awq_gemm(torch.from_numpy(x).to(dev), qw, sc, qz, out=out)
    ms = sample_idx(M, 24, seed=M, must=(0, 1, M // 2))
    y = to_np(out[torch.from_numpy(ms).to(dev)])
    assert not np.isnan(y).any(), "output not fully written"
    assert np.all(y[0] == 0), "an all-zero X row must give exactly 0"
    # exact reference, 4096 columns at a time (integers in fp64: exact)
    xs = x[ms].astype(np.float64)
    for n0 in range(0, N, 4096):
        n1 = min(N, n0 + 4096)
        wq = q[n0:n1].astype(np.float64) - np.repeat(z[n0:n1].astype(np.float64), 128, axis=1)
        exact = (xs @ wq.T) / 8.0
        assert np.abs(exact).max() < 65504
        got = y[:, n0:n1]
        bad = got.view(np.uint16) != exact.astype(np.float16).view(np.uint16)
        assert not bad.any(), (name, M, int(bad.sum()), np.argwhere(bad)[:4].tolist())
