"""GPU parity of the W4A8 stage against the oracle.

* w4a8_quant_act: no-norm mode bit-exact (the fp32 decisions have one defined
  sequence); RMSNorm mode equal except at near-ties, where the kernel's fp32 sum of
  squares (a different summation order than the oracle's exact sum) may move the
  value across a .5 boundary; there the code may differ by 1.
* w4a8_gemm_i32: the int32 accumulators, bit-exact, fed the oracle's xq and packed
  weights (per-channel and two-level g128), small ragged shapes and the full shapes.
* w4a8_gemm: fp16 outputs within the normalized 2e-3 bound.
* w4a8_silu_mul_quant: codes equal except at near-ties (the kernel's y is fp32, the
  oracle's fp64), where they may differ by 1; s_a within 1e-6 relative.
"""
import numpy as np
import pytest
import torch

import oracle.ref as ora
import synth
import w4a16_gemm_amd as w4
from gpu_util import TOL, announce, device, normalized_error, sample_idx, to_np

pytestmark = pytest.mark.gpu

# |t_gpu - t_oracle| bound for the RMSNorm-mode quantization argument t = y * 127 / max|y|:
# fp32 sum of K squares (relative error <= ~log2(K) * 2^-24 after pairwise/tree
# reduction, ~1e-6 bounded generously), two fp32 products and the division give a
# relative error below ~2e-6, i.e. |dt| <= 127 * 2e-6 = 2.5e-4.
NEAR_TIE = 2.5e-4


# widths cover every launch variant: 256 threads with 1, 2, 4 and 8 vectors of 8 per
# thread, 128 threads with 5 (K = 5120), 1024 threads with 4, and the streaming variant
@pytest.mark.parametrize("M,K", [(1, 128), (3, 4096), (7, 5120), (64, 13824), (300, 5120), (5, 20096), (2, 40064),
                                 (4096, 5120), (4096, 13824)])
def test_quant_act_no_norm_bit_exact(M, K):
    dev = device()
    announce(f"quant_act no-norm M={M} K={K}")
    x = synth.make_activations(M, K, seed=M, rms_spread=True)
    x[0, :] = 0  # a zero row: s_a = 1, codes 0
    xq, sa = w4.w4a8_quant_act(x.to(dev), None)
    torch.cuda.synchronize()
    rxq, rsa, _ = ora.w4a8_quant_act_ref(x.numpy(), None)
    assert np.array_equal(to_np(xq), rxq)
    assert np.array_equal(to_np(sa).view(np.uint32), rsa.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 128), (3, 4096), (16, 5120), (256, 5120), (4096, 5120), (33, 13824), (5, 20096),
                                 (2, 40064)])
def test_quant_act_rmsnorm_near_ties_only(M, K):
    dev = device()
    announce(f"quant_act rmsnorm M={M} K={K}")
    inp = synth.make_linear(M, 8, K, seed=M + 1, rms_spread=True, with_gamma=True)
    x, gamma = inp.x, inp.gamma
    if M > 1:
        x[1, :] = 0
    xq, sa = w4.w4a8_quant_act(x.to(dev), gamma.to(dev), 1e-5)
    torch.cuda.synchronize()
    rxq, rsa, t = ora.w4a8_quant_act_ref(x.numpy(), gamma.numpy(), 1e-5)
    gq = to_np(xq).astype(np.int64)
    diff = np.abs(gq - rxq.astype(np.int64))
    assert diff.max() <= 1
    frac = np.abs(np.abs(t - np.trunc(t)) - 0.5)
    assert np.all(frac[diff == 1] < NEAR_TIE), float(frac[diff == 1].max())
    assert (diff == 1).mean() < 1e-3
    rel = np.abs(to_np(sa).astype(np.float64) / rsa.astype(np.float64) - 1)
    assert rel.max() <= 2e-6
    assert np.all(np.abs(gq).max(axis=1)[np.abs(x.numpy()).max(axis=1) > 0] == 127)


# |t_gpu - t_oracle| bound for the SiLU-gated quantization argument t = y * 127 / max|y|,
# in units u = 2^-24 of relative error.  Kernel: exp(-g) from the 1-ulp hardware 2^x
# (2u) times the first-order residual factor (1u) and its product (1u): 4u; 1 + e: 5u;
# the 1-ulp reciprocal: 7u; g * u and the last product: y within 9u of the exact value,
# amax likewise, fp32(127 / amax) 10u, t = y * inv 20u.  Oracle: fp32(y), amax, the
# division and the product, about 4u.  |dt| <= 127 * 24u = 1.8e-4; bounded at 2.5e-4.
NEAR_TIE_SILU = 2.5e-4


# widths cover every launch variant: 256 threads with 1, 2, 4 and 8 vectors per thread,
# 128 threads with 5 (I = 5120), 1024 threads with 4 and 8, and the streaming variant;
# I = 8 leaves 255 threads idle
@pytest.mark.parametrize("M,I", [(1, 8), (2, 1000), (3, 2056), (64, 5120), (1, 13824), (16, 13824),
                                 (257, 13824), (5, 20000), (4, 40000), (3, 70008), (4096, 13824)])
def test_silu_mul_quant_near_ties_only(M, I):
    dev = device()
    announce(f"silu_mul_quant M={M} I={I}")
    gu = synth.make_activations(M, 2 * I, seed=M + I, rms_spread=True)
    gu[0, :I] = 0  # zero gate row: y = 0, s_a = 1, codes 0
    if M > 2:
        gu[1, :I] = -65504.0  # silu -> -0: a zero row from the exp overflow side
        gu[2, : I // 2] = 65504.0  # silu(g) = g: the largest |y| in the test
    if M > 4:
        gu[3, :I] = -50.0  # with |up| <= 1: max|y| ~ 1e-20, a live row of tiny values
        gu[3, I:] = gu[3, I:].clamp(-1, 1)
        gu[4, :I] = -45.0  # max|y| ~ 1e-18: a live row of tiny values
    if M > 6:
        gu[5, :I] = -90.0  # |up| in [4, 8]: max|y| ~ 5.9e-37, live; s_a ~ 4.6e-39 is subnormal
        gu[5, I:] = 4.0 + 4.0 * torch.rand(I, generator=torch.Generator().manual_seed(M)).to(torch.float16)
        gu[5, I] = 8.0
        gu[6, :I] = -90.0  # |up| <= 1: max|y| <= 7.4e-38, fp32(127 / max|y|) overflows: a zero row
        gu[6, I:] = gu[6, I:].clamp(-1, 1)
    xq, sa = w4.w4a8_silu_mul_quant(gu.to(dev))
    torch.cuda.synchronize()
    rxq, rsa, t = ora.silu_mul_quant_ref(gu.numpy())
    gq = to_np(xq).astype(np.int64)
    diff = np.abs(gq - rxq.astype(np.int64))
    assert diff.max() <= 1
    frac = np.abs(np.abs(t - np.trunc(t)) - 0.5)
    assert np.all(frac[diff == 1] < NEAR_TIE_SILU), float(frac[diff == 1].max())
    assert (diff == 1).mean() < 1e-3
    rel = np.abs(to_np(sa).astype(np.float64) / rsa.astype(np.float64) - 1)
    normal = rsa >= np.finfo(np.float32).tiny
    assert rel[normal].max() <= 1e-6
    # subnormal s_a: the oracle's and the kernel's roundings are each up to half a
    # subnormal step (3e-7 of 4.6e-39) next to the kernel's ~5e-7 in max|y|
    assert rel[~normal].max(initial=0.0) <= 4e-6
    assert float(to_np(sa)[0]) == 1.0 and not gq[0].any()
    if M > 2:
        assert float(to_np(sa)[1]) == 1.0 and not gq[1].any()
    if M > 4:
        assert np.abs(gq[3]).max() == 127 and np.abs(gq[4]).max() == 127
    if M > 6:
        assert 0.0 < float(to_np(sa)[5]) < np.finfo(np.float32).tiny and np.abs(gq[5]).max() == 127
        assert float(to_np(sa)[6]) == 1.0 and not gq[6].any()
    live = np.abs(t).max(axis=1) > 0
    assert np.all(np.abs(gq).max(axis=1)[live] == 127)


def test_silu_mul_quant_bound_call_repeats():
    dev = device()
    announce("silu_mul_quant bound call")
    M, I = 16, 13824
    gu = synth.make_activations(M, 2 * I, seed=5, rms_spread=True).to(dev)
    xq = torch.empty((M, I), dtype=torch.int8, device=dev)
    sa = torch.empty((M,), dtype=torch.float32, device=dev)
    call = w4.bind_w4a8_silu_mul_quant(gu, xq, sa)
    call()
    torch.cuda.synchronize()
    first = (to_np(xq).copy(), to_np(sa).copy())
    xq.fill_(0)
    sa.fill_(0)
    call()
    torch.cuda.synchronize()
    rq, rs = w4.w4a8_silu_mul_quant(gu)
    torch.cuda.synchronize()
    for a in (first, (to_np(xq), to_np(sa))):
        assert np.array_equal(a[0], to_np(rq)) and np.array_equal(a[1].view(np.uint32), to_np(rs).view(np.uint32))


def _oracle_w4a8(w16, group, dev):
    q, cs, gs = ora.quantize_w4a8(w16, group)
    qw, cs2, gs_gn = ora.pack_w4a8(q, cs, gs)
    tens = [torch.from_numpy(np.ascontiguousarray(qw)).to(dev),
            None if gs_gn is None else torch.from_numpy(gs_gn).to(dev),
            torch.from_numpy(cs2).to(dev)]
    return q, cs2, gs, tens


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (5, 200, 384), (16, 1000, 1024), (33, 96, 2048), (64, 256, 640),
                                   (100, 300, 1280), (257, 520, 2048), (512, 512, 5120)])
def test_w4a8_gemm_small(group, M, N, K):
    dev = device()
    announce(f"w4a8 small M={M} N={N} K={K} group={group}")
    inp = synth.make_linear(M, N, K, seed=M * 3 + N, outliers=True, rms_spread=True, with_gamma=True)
    q, cs, gs, (qw, gsd, csd) = _oracle_w4a8(inp.w.numpy(), group, dev)
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    xqd, sad = torch.from_numpy(xq).to(dev), torch.from_numpy(sa).to(dev)
    acc = to_np(w4.w4a8_gemm_i32(xqd, qw, gsd, group, N=N))
    racc = ora.w4a8_acc_ref(xq, q, gs, 128)
    assert np.abs(racc).max() < 2**31
    assert np.array_equal(acc.astype(np.int64), racc)
    out = w4.w4a8_gemm(xqd, sad, qw, gsd, csd, group)
    torch.cuda.synchronize()
    y = to_np(out).astype(np.float64)
    yr = ora.w4a8_linear_ref(racc, sa, cs)
    qs = q.astype(np.float64) * (1 if gs is None else np.repeat(gs.astype(np.float64), 128, axis=1))
    wn = np.linalg.norm(qs, axis=1) * cs.astype(np.float64)
    xn = np.linalg.norm(xq.astype(np.float64), axis=1) * sa.astype(np.float64)
    assert normalized_error(y, yr, xn, wn) <= TOL


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("bm_depth", ["32,1", "32,4", "64,1", "64,3", "64,4", "128,1", "64,0", "128,0", "64,5", "128,5"])
@pytest.mark.parametrize("M,N,K,target", [(70, 300, 1280, "1"), (200, 520, 2048, "128"), (40, 129, 128, "1"),
                                          (300, 260, 1152, "4")])
def test_w4a8_gemm_tiles_and_depths(group, bm_depth, M, N, K, target, monkeypatch):
    """Each compiled row-tile height and prefetch depth of the int8 GEMM (rotating
    register sets: steady state plus a tail shorter than the sets), split and unsplit,
    ragged M and N, one group (K = 128): int32 accumulators bit-exact."""
    dev = device()
    bm, depth = bm_depth.split(",")
    monkeypatch.setenv("W4_W4A8_BM", bm)
    monkeypatch.setenv("W4_W4A8_DEPTH", depth)
    monkeypatch.setenv("W4_W4A8_SPLIT_TARGET", target)
    announce(f"w4a8 bm={bm} depth={depth} M={M} N={N} K={K} group={group}")
    inp = synth.make_linear(M, N, K, seed=M + N + int(depth), outliers=True, rms_spread=True, with_gamma=True)
    q, cs, gs, (qw, gsd, csd) = _oracle_w4a8(inp.w.numpy(), group, dev)
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    acc = to_np(w4.w4a8_gemm_i32(torch.from_numpy(xq).to(dev), qw, gsd, group, N=N))
    assert np.array_equal(acc.astype(np.int64), ora.w4a8_acc_ref(xq, q, gs, 128))


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("M,N,K,div,parts", [(600, 1000, 2048, 32, 2), (300, 520, 1280, 64, 4)])
@pytest.mark.parametrize("depth", ["1", "0", "5"])
def test_w4a8_gemm_tail_split(group, M, N, K, div, parts, depth, monkeypatch):
    """The 128-row int8 GEMM with the last tiles split over their groups (the remainder
    of the tile count over the resident workgroups; the slot count scaled down through
    the tuning variables so small shapes reach it): int32 accumulators bit-exact, fp16
    outputs within 2e-3, and a second call on the same workspace."""
    dev = device()
    monkeypatch.setenv("W4_W4A8_SPLIT_TARGET", "1")
    monkeypatch.setenv("W4_W4A8_TAIL", "1")
    monkeypatch.setenv("W4_W4A8_BM", "128")
    monkeypatch.setenv("W4_W4A8_DEPTH", depth)
    monkeypatch.setenv("W4_W4A8_SLOTS_DIV", str(div))
    monkeypatch.setenv("W4_W4A8_TAIL_PARTS", str(parts))
    tiles = -(-M // 128) * -(-N // 256)
    rem = tiles % (512 // div)
    assert w4.w4a8_gemm_workspace_bytes(M, N, K, group) == 16384 + rem * parts * 128 * 256 * 4
    announce(f"w4a8 tail split M={M} N={N} K={K} group={group} tiles={tiles} parts={parts}")
    inp = synth.make_linear(M, N, K, seed=M * 5 + N, outliers=True, rms_spread=True, with_gamma=True)
    q, cs, gs, (qw, gsd, csd) = _oracle_w4a8(inp.w.numpy(), group, dev)
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    xqd, sad = torch.from_numpy(xq).to(dev), torch.from_numpy(sa).to(dev)
    racc = ora.w4a8_acc_ref(xq, q, gs, 128)
    yr = ora.w4a8_linear_ref(racc, sa, cs)
    qs = q.astype(np.float64) * (1 if gs is None else np.repeat(gs.astype(np.float64), 128, axis=1))
    wn = np.linalg.norm(qs, axis=1) * cs.astype(np.float64)
    xn = np.linalg.norm(xq.astype(np.float64), axis=1) * sa.astype(np.float64)
    for _ in range(2):
        acc = to_np(w4.w4a8_gemm_i32(xqd, qw, gsd, group, N=N))
        assert np.array_equal(acc.astype(np.int64), racc)
        y = to_np(w4.w4a8_gemm(xqd, sad, qw, gsd, csd, group)).astype(np.float64)
        assert normalized_error(y, yr, xn, wn) <= TOL


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("M", [1, 16, 256, 4096])
def test_w4a8_full_size_sampled(group, M):
    """C5 shapes (K = 5120, N = 13824) end to end on the GPU: pack, quant_act (RMSNorm),
    GEMM; accumulators bit-exact on the oracle's xq; fp16 outputs within 2e-3."""
    dev = device()
    N, K = 13824, 5120
    announce(f"w4a8 full M={M} group={group}")
    inp = synth.make_linear(M, N, K, seed=0, outliers=True, rms_spread=True, with_gamma=True)
    qw, gs, cs = w4.w4a8_pack(inp.w.to(dev), group)
    xq, sa = w4.w4a8_quant_act(inp.x.to(dev), inp.gamma.to(dev))
    y = w4.w4a8_gemm(xq, sa, qw, gs, cs, group)
    rxq, rsa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    acc = w4.w4a8_gemm_i32(torch.from_numpy(rxq).to(dev), qw, gs, group, N=N)
    torch.cuda.synchronize()
    ms = sample_idx(M, 48, seed=M)
    ns = sample_idx(N, 256, seed=7, must=range(0, 32))
    q, rcs, rgs = ora.quantize_w4a8(inp.w.numpy()[ns], group)
    racc = ora.w4a8_acc_ref(rxq[ms], q, rgs, 128)
    assert np.array_equal(to_np(acc)[np.ix_(ms, ns)].astype(np.int64), racc)
    # fp16 outputs of the all-GPU chain against the oracle chain
    yr = ora.w4a8_linear_ref(racc, rsa[ms], rcs)
    qs = q.astype(np.float64) * (1 if rgs is None else np.repeat(rgs.astype(np.float64), 128, axis=1))
    wn = np.linalg.norm(qs, axis=1) * rcs.astype(np.float64)
    xn = np.linalg.norm(rxq[ms].astype(np.float64), axis=1) * rsa[ms].astype(np.float64)
    err = normalized_error(to_np(y)[np.ix_(ms, ns)].astype(np.float64), yr, xn, wn)
    assert err <= TOL, err


@pytest.mark.parametrize("group", [-1, 128])
def test_w4a8_down_shape_default_tail(group):
    """The down projection at prefill (M = 4096, K = 13824, N = 5120): 640 128 x 256 tiles
    on 512 resident workgroups, so the default plan splits the 128 tiles of the last round
    over their groups; int32 accumulators bit-exact on sampled outputs that include rows
    and columns of those tiles (the last row block group: rows 3072.., columns 1024..)."""
    dev = device()
    M, N, K = 4096, 5120, 13824
    assert w4.w4a8_gemm_workspace_bytes(M, N, K, group) == 16384 + 128 * 2 * 128 * 256 * 4
    announce(f"w4a8 down shape default tail M={M} group={group}")
    inp = synth.make_linear(M, N, K, seed=3, outliers=True, rms_spread=True, with_gamma=True)
    qw, gs, cs = w4.w4a8_pack(inp.w.to(dev), group)
    rxq, rsa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    xqd, sad = torch.from_numpy(rxq).to(dev), torch.from_numpy(rsa).to(dev)
    acc = w4.w4a8_gemm_i32(xqd, qw, gs, group, N=N)
    y = w4.w4a8_gemm(xqd, sad, qw, gs, cs, group)
    torch.cuda.synchronize()
    ms = sample_idx(M, 48, seed=11, must=list(range(0, 8)) + list(range(4088, 4096)))
    ns = sample_idx(N, 256, seed=12, must=list(range(0, 16)) + list(range(5104, 5120)))
    q, rcs, rgs = ora.quantize_w4a8(inp.w.numpy()[ns], group)
    racc = ora.w4a8_acc_ref(rxq[ms], q, rgs, 128)
    assert np.array_equal(to_np(acc)[np.ix_(ms, ns)].astype(np.int64), racc)
    yr = ora.w4a8_linear_ref(racc, rsa[ms], rcs)
    qs = q.astype(np.float64) * (1 if rgs is None else np.repeat(rgs.astype(np.float64), 128, axis=1))
    wn = np.linalg.norm(qs, axis=1) * rcs.astype(np.float64)
    xn = np.linalg.norm(rxq[ms].astype(np.float64), axis=1) * rsa[ms].astype(np.float64)
    err = normalized_error(to_np(y)[np.ix_(ms, ns)].astype(np.float64), yr, xn, wn)
    assert err <= TOL, err


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("tiles", ["1", "2", "4", "off"])
@pytest.mark.parametrize("M,N,K", [(1, 200, 1024), (7, 1000, 2048), (16, 130, 13824), (3, 64, 128)])
def test_w4a8_skinny_variants(group, tiles, M, N, K, monkeypatch):
    """The M <= 16 W4A8 kernel at each tile width (forced through its tuning variable),
    ragged N, one group (K = 128) and split K; 'off' forces the tiled GEMM.  int32
    accumulators bit-exact on the oracle's xq."""
    dev = device()
    if tiles == "off":
        monkeypatch.setenv("W4_W4A8_SKINNY", "0")
    else:
        monkeypatch.setenv("W4_W4A8_TILES", tiles)
    announce(f"w4a8 skinny tiles={tiles} M={M} N={N} K={K} group={group}")
    inp = synth.make_linear(M, N, K, seed=M * 11 + N, outliers=True, rms_spread=True, with_gamma=True)
    q, cs, gs, (qw, gsd, csd) = _oracle_w4a8(inp.w.numpy(), group, dev)
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    xqd = torch.from_numpy(xq).to(dev)
    acc = to_np(w4.w4a8_gemm_i32(xqd, qw, gsd, group, N=N))
    assert np.array_equal(acc.astype(np.int64), ora.w4a8_acc_ref(xq, q, gs, 128))
    out = to_np(w4.w4a8_gemm(xqd, torch.from_numpy(sa).to(dev), qw, gsd, csd, group)).astype(np.float64)
    yr = ora.w4a8_linear_ref(ora.w4a8_acc_ref(xq, q, gs, 128), sa, cs)
    qs = q.astype(np.float64) * (1 if gs is None else np.repeat(gs.astype(np.float64), 128, axis=1))
    wn = np.linalg.norm(qs, axis=1) * cs.astype(np.float64)
    xn = np.linalg.norm(xq.astype(np.float64), axis=1) * sa.astype(np.float64)
    assert normalized_error(out, yr, xn, wn) <= TOL


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.choice([1, 2, 5, 16, 17, 33, 64, 100, 257])), int(rng.integers(1, 600)),
             128 * int(rng.integers(1, 33))) for _ in range(n)]


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("M,N,K", _random_shapes(16, seed=2027))
def test_w4a8_random_shapes(group, M, N, K):
    """Seeded random shapes across the skinny / GEMM boundary and split-K choices: int32
    accumulators bit-exact on the oracle's xq."""
    dev = device()
    announce(f"w4a8 random M={M} N={N} K={K} group={group}")
    inp = synth.make_linear(M, N, K, seed=M * 17 + N + K, outliers=True, rms_spread=True, with_gamma=True)
    q, cs, gs, (qw, gsd, csd) = _oracle_w4a8(inp.w.numpy(), group, dev)
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    acc = to_np(w4.w4a8_gemm_i32(torch.from_numpy(xq).to(dev), qw, gsd, group, N=N))
    assert np.array_equal(acc.astype(np.int64), ora.w4a8_acc_ref(xq, q, gs, 128))


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("M", [1, 4, 16, 256])
def test_down_projection_chain_full_size(group, M):
    """The W4A8 MLP tail at its real shape: fused gate+up output [M, 2 x 13824] ->
    silu_mul_quant -> down projection (K = 13824, N = 5120) on the int8 GEMM.  Codes
    within the SiLU near-tie rule; accumulators on the GPU's codes bit-exact against the
    oracle's integer sum; fp16 outputs within 2e-3 of the oracle chain."""
    dev = device()
    I, N = 13824, 5120
    announce(f"down-projection chain M={M} group={group}")
    gu = synth.make_activations(M, 2 * I, seed=M + 77, rms_spread=True)
    w = synth.make_linear(0, N, I, seed=5, outliers=True).w
    qw, gs, cs = w4.w4a8_pack(w.to(dev), group)
    xq, sa = w4.w4a8_silu_mul_quant(gu.to(dev))
    y = w4.w4a8_gemm(xq, sa, qw, gs, cs, group)
    acc = w4.w4a8_gemm_i32(xq, qw, gs, group, N=N)
    torch.cuda.synchronize()
    rxq, rsa, t = ora.silu_mul_quant_ref(gu.numpy())
    gq = to_np(xq).astype(np.int64)
    diff = np.abs(gq - rxq.astype(np.int64))
    assert diff.max() <= 1
    assert np.all(np.abs(np.abs(t - np.trunc(t)) - 0.5)[diff == 1] < NEAR_TIE_SILU)
    ms = sample_idx(M, 24, seed=M)
    ns = sample_idx(N, 192, seed=11, must=range(0, 16))
    q, rcs, rgs = ora.quantize_w4a8(w.numpy()[ns], group)
    racc = ora.w4a8_acc_ref(gq[ms], q, rgs, 128)
    assert np.array_equal(to_np(acc)[np.ix_(ms, ns)].astype(np.int64), racc)
    yr = ora.w4a8_linear_ref(ora.w4a8_acc_ref(rxq[ms], q, rgs, 128), rsa[ms], rcs)
    qs = q.astype(np.float64) * (1 if rgs is None else np.repeat(rgs.astype(np.float64), 128, axis=1))
    wn = np.linalg.norm(qs, axis=1) * rcs.astype(np.float64)
    xn = np.linalg.norm(rxq[ms].astype(np.float64), axis=1) * rsa[ms].astype(np.float64)
    err = normalized_error(to_np(y)[np.ix_(ms, ns)].astype(np.float64), yr, xn, wn)
    assert err <= TOL, err
