"""GPU: the int8 GEMMs at their largest K (131072) with extreme operands, where the int32
accumulators come closest to overflowing, and the W4A16 path at a long K.  Operands are
built directly in the packed formats (not through the quantizers) so every code sits at
its extreme; expected values are closed forms.

* W4A8 per-channel: xq = 127, q = -8 everywhere.  The kernel sums 127 * (16 q) = -16256
  per k, -2 130 706 432 over K (inside int32), and the exact shift by 4 gives
  127 * -8 * K = -133 169 152.
* W4A8 two-level: xq = -127, q = 7, s_g = 18 (q s_g = 126): 127 * -126 * K = -2 097 414 144.
* W8A8: xq = q = -127: 127^2 * K = 2 114 060 288.
* Any K above 131072 is refused (W4_ERR_UNSUPPORTED) before a kernel runs.
* X of more than 2^31 elements (M = 16400, K = 131072): the W4A16 and W4A8 GEMMs fall
  back from their 32-bit-offset direct-to-LDS loops to 64-bit offsets; one-hot X rows
  make every sampled output a single weight element, compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle.ref as ora
import synth
import w4a16_gemm_amd as w4
from gpu_util import TOL, announce, device, normalized_error, sample_idx, to_np

pytestmark = pytest.mark.gpu

KMAX = 131072


@pytest.mark.parametrize("M,N", [(1, 64), (3, 40), (17, 48)])
def test_w4a8_per_channel_extreme_at_max_k(M, N):
    dev = device()
    announce(f"w4a8 per-channel extreme K={KMAX} M={M} N={N}")
    q = np.full((N, KMAX), -8, np.int64)
    qw, cs, _ = ora.pack_w4a8(q, np.ones(N, np.float16), None)
    xq = torch.full((M, KMAX), 127, dtype=torch.int8, device=dev)
    acc = to_np(w4.w4a8_gemm_i32(xq, torch.from_numpy(qw).to(dev), None, -1, N=N))
    assert np.all(acc.astype(np.int64) == 127 * -8 * KMAX)


@pytest.mark.parametrize("M,N", [(1, 64), (16, 40)])
def test_w4a8_two_level_extreme_at_max_k(M, N):
    dev = device()
    announce(f"w4a8 two-level extreme K={KMAX} M={M} N={N}")
    q = np.full((N, KMAX), 7, np.int64)
    gs = np.full((N, KMAX // 128), 18, np.int8)
    qw, cs, gs_gn = ora.pack_w4a8(q, np.ones(N, np.float16), gs)
    xq = torch.full((M, KMAX), -127, dtype=torch.int8, device=dev)
    acc = to_np(w4.w4a8_gemm_i32(xq, torch.from_numpy(qw).to(dev), torch.from_numpy(gs_gn).to(dev), 128, N=N))
    assert np.all(acc.astype(np.int64) == -127 * 126 * KMAX)


@pytest.mark.parametrize("M,N", [(1, 64), (16, 40), (65, 32)])
def test_w8a8_extreme_at_max_k(M, N):
    dev = device()
    announce(f"w8a8 extreme K={KMAX} M={M} N={N}")
    q = np.full((N, KMAX), -127, np.int8)
    xq = torch.full((M, KMAX), -127, dtype=torch.int8, device=dev)
    acc = to_np(w4.w8a8_gemm_i32(xq, torch.from_numpy(ora.tile_w8a8(q)).to(dev), N))
    assert np.all(acc.astype(np.int64) == 127 * 127 * KMAX)


def test_int8_gemms_refuse_k_beyond_range():
    dev = device()
    K = KMAX + 128
    xq = torch.zeros((1, K), dtype=torch.int8, device=dev)
    qw8 = torch.zeros(w4.w8a8_qweight_shape(16, K), dtype=torch.int8, device=dev)
    with pytest.raises(w4.W4Error, match="131072"):
        w4.w8a8_gemm_i32(xq, qw8, 16)
    qw4 = torch.zeros(w4.qweight_shape(16, K), dtype=torch.int32, device=dev)
    with pytest.raises(w4.W4Error, match="131072"):
        w4.w4a8_gemm_i32(xq, qw4, None, -1, N=16)


@pytest.mark.parametrize("M", [1, 16, 100])
def test_w4a16_long_k(M):
    """K = 65536 (512 groups): the skinny kernels' and the GEMM's split-K at a long K,
    sampled outputs against the oracle."""
    dev = device()
    N, K = 512, 65536
    announce(f"w4a16 long K={K} M={M}")
    inp = synth.make_linear(M, N, K, seed=M + 3, outliers=True, rms_spread=True)
    qw, sc, qz = w4.awq_pack(inp.w.to(dev))
    y = to_np(w4.awq_gemm(inp.x.to(dev), qw, sc, qz)).astype(np.float64)
    ns = sample_idx(N, 64, seed=M)
    ref = ora.awq_reference(inp.w.numpy()[ns], inp.x.numpy(), 128)
    err = normalized_error(y[:, ns], ref["y"], np.linalg.norm(inp.x.numpy().astype(np.float64), axis=1),
                           np.linalg.norm(ref["w_deq"], axis=1))
    assert err <= TOL, err


# X beyond 2^31 elements: the direct-to-LDS pipelines form X offsets in 32 bits, so the
# plans fall back to the register-staged loop (64-bit offsets) when M K >= 2^31.  One 1
# per X row, at a row-specific k: every output of row m is then a single weight element,
# (q - z) / 8 exactly (W4A16, scales 2^-3) or q (W4A8 per-channel), so a wrong row offset
# anywhere (rows past 2^31 / K = 16384 included) changes the sampled outputs.
M_BIG, K_BIG, N_BIG = 16400, 131072, 512


def _one_hot_rows(M, K, dtype, dev):
    kk = (np.arange(M, dtype=np.int64) * 977 + 13) % K
    x = torch.zeros((M, K), dtype=dtype, device=dev)
    x[torch.arange(M, device=dev), torch.from_numpy(kk).to(dev)] = 1
    return x, kk


def _big_rows(M):
    rng = np.random.default_rng(5)
    return np.unique(np.concatenate([[0, 1, M // 2, 16383, 16384, 16385, M - 1], rng.integers(0, M, 9)]))


def test_w4a16_x_beyond_32bit_offsets():
    dev = device()
    M, K, N = M_BIG, K_BIG, N_BIG
    assert M * K >= 2**31
    announce(f"w4a16 X of {M * K} elements M={M} K={K} N={N}")
    rng = np.random.default_rng(21)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    words = w4.w4_pack_codes(torch.from_numpy(q).to(dev))
    zw = w4.w4_pack_codes(torch.from_numpy(z).to(dev))
    s = torch.full((N, K // 128), 0.125, dtype=torch.float16, device=dev)
    qw, sc, qz = w4.awq_import_plain(words, s, zw, 128, "rows")
    del words, zw, s
    x, kk = _one_hot_rows(M, K, torch.float16, dev)
    y = w4.awq_gemm(x, qw, sc, qz)
    torch.cuda.synchronize()
    rows = _big_rows(M)
    got = to_np(y[torch.from_numpy(rows).to(dev)])
    del x, y, qw, sc, qz
    torch.cuda.empty_cache()
    exact = (q[:, kk[rows]].T.astype(np.float64) - z[:, kk[rows] // 128].T.astype(np.float64)) / 8.0
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16))


def test_w4a8_x_beyond_32bit_offsets():
    dev = device()
    M, K, N = M_BIG, K_BIG, N_BIG
    announce(f"w4a8 xq of {M * K} bytes M={M} K={K} N={N}")
    rng = np.random.default_rng(22)
    q = rng.integers(-8, 8, size=(N, K), dtype=np.int64)
    words = w4.w4_pack_codes(torch.from_numpy((q + 8).astype(np.uint8)).to(dev))
    qw, _ = w4.w4a8_import_plain(words, None, -1, "rows")
    del words
    xq, kk = _one_hot_rows(M, K, torch.int8, dev)
    acc = w4.w4a8_gemm_i32(xq, qw, None, -1, N=N)
    torch.cuda.synchronize()
    rows = _big_rows(M)
    got = to_np(acc[torch.from_numpy(rows).to(dev)])
    del xq, acc, qw
    torch.cuda.empty_cache()
    assert np.array_equal(got.astype(np.int64), q[:, kk[rows]].T)
