"""GPU parity of the W8A8 path (per-channel int8 weights, per-token int8 activations)
against the oracle.

* w8a8_pack: tiled int8 codes (padding rows included) and fp16 scales bit-exact
  (small ragged shapes; full shapes sampled);
* w8a8_gemm_i32: the int32 accumulators bit-exact on the oracle's xq and codes, through
  the M <= 16 kernel at each tile width and the tiled GEMM at each row-tile size, with
  and without split K, ragged N, one group (K = 128), the full shapes, and seeded random
  shapes;
* w8a8_gemm: fp16 outputs within the normalized 2e-3 bound (the accumulator is exact;
  only the two fp32 products and the fp16 output round).
"""
import numpy as np
import pytest
import torch

import oracle.ref as ora
import synth
import w4a16_gemm_amd as w4
from gpu_util import TOL, announce, device, normalized_error, sample_idx, to_np

pytestmark = pytest.mark.gpu


def _check_fp16(y, xq, sa, q, cs):
    racc = ora.w4a8_acc_ref(xq, q, None, 128)
    yr = ora.w4a8_linear_ref(racc, sa, cs)
    wn = np.linalg.norm(q.astype(np.float64), axis=1) * cs.astype(np.float64)
    xn = np.linalg.norm(xq.astype(np.float64), axis=1) * sa.astype(np.float64)
    err = normalized_error(y, yr, xn, wn)
    assert err <= TOL, err


@pytest.mark.parametrize("N,K", [(64, 128), (13, 256), (200, 1024), (1000, 5120)])
def test_w8a8_pack_bit_exact(N, K):
    dev = device()
    announce(f"w8a8_pack N={N} K={K}")
    w = synth.make_linear(0, N, K, seed=N + K, outliers=True).w
    qw, cs = w4.w8a8_pack(w.to(dev))
    torch.cuda.synchronize()
    q, s = ora.quantize_w8a8(w.numpy())
    assert np.array_equal(to_np(qw), ora.tile_w8a8(q))
    assert np.array_equal(to_np(cs).view(np.uint16), s.view(np.uint16))


SHAPES = [(1, 64, 128), (5, 200, 384), (16, 1000, 1024), (33, 96, 2048), (64, 256, 640), (100, 300, 1280),
          (257, 520, 2048), (512, 512, 5120)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w8a8_gemm_small(M, N, K):
    dev = device()
    announce(f"w8a8 small M={M} N={N} K={K} ws={w4.w8a8_gemm_workspace_bytes(M, N, K)}")
    inp = synth.make_linear(M, N, K, seed=M * 3 + N, outliers=True, rms_spread=True, with_gamma=True)
    q, cs = ora.quantize_w8a8(inp.w.numpy())
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    xqd, sad = torch.from_numpy(xq).to(dev), torch.from_numpy(sa).to(dev)
    qd, csd = torch.from_numpy(ora.tile_w8a8(q)).to(dev), torch.from_numpy(cs).to(dev)
    acc = to_np(w4.w8a8_gemm_i32(xqd, qd, N))
    racc = ora.w4a8_acc_ref(xq, q, None, 128)
    assert np.abs(racc).max() < 2**31
    assert np.array_equal(acc.astype(np.int64), racc)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    y = to_np(w4.w8a8_gemm(xqd, sad, qd, csd, out=out)).astype(np.float64)
    assert np.all(np.isfinite(y)), "output not fully written"
    _check_fp16(y, xq, sa, q, cs)


@pytest.mark.parametrize("tiles", ["1", "2", "4", "off"])
@pytest.mark.parametrize("M,N,K", [(1, 200, 1024), (7, 1000, 2048), (16, 130, 13824), (3, 64, 128)])
def test_w8a8_skinny_variants(tiles, M, N, K, monkeypatch):
    """The M <= 16 kernel at each tile width (forced through its tuning variable), ragged
    N, one group and split K; 'off' forces the tiled GEMM."""
    dev = device()
    if tiles == "off":
        monkeypatch.setenv("W4_W4A8_SKINNY", "0")
    else:
        monkeypatch.setenv("W4_W4A8_TILES", tiles)
    announce(f"w8a8 skinny tiles={tiles} M={M} N={N} K={K}")
    inp = synth.make_linear(M, N, K, seed=M * 11 + N, outliers=True, rms_spread=True, with_gamma=True)
    q, cs = ora.quantize_w8a8(inp.w.numpy())
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    xqd, qd = torch.from_numpy(xq).to(dev), torch.from_numpy(ora.tile_w8a8(q)).to(dev)
    acc = to_np(w4.w8a8_gemm_i32(xqd, qd, N))
    assert np.array_equal(acc.astype(np.int64), ora.w4a8_acc_ref(xq, q, None, 128))


@pytest.mark.parametrize("bm_depth", ["32,1", "32,4", "64,1", "64,3", "64,4", "128,1", "64,0", "128,0", "64,5", "128,5"])
@pytest.mark.parametrize("M,N,K,target", [(70, 300, 1280, "1"), (200, 520, 2048, "128"), (40, 129, 128, "1"),
                                          (300, 260, 1152, "4")])
def test_w8a8_gemm_tiles_and_depths(bm_depth, M, N, K, target, monkeypatch):
    """Each compiled row-tile height and prefetch depth of the int8 GEMM on W8A8
    weights, split and unsplit, ragged shapes: int32 accumulators bit-exact."""
    dev = device()
    bm, depth = bm_depth.split(",")
    monkeypatch.setenv("W4_W4A8_BM", bm)
    monkeypatch.setenv("W4_W4A8_DEPTH", depth)
    monkeypatch.setenv("W4_W4A8_SPLIT_TARGET", target)
    announce(f"w8a8 bm={bm} depth={depth} M={M} N={N} K={K}")
    inp = synth.make_linear(M, N, K, seed=M + N + int(depth), outliers=True, rms_spread=True, with_gamma=True)
    q, cs = ora.quantize_w8a8(inp.w.numpy())
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    qd = torch.from_numpy(ora.tile_w8a8(q)).to(dev)
    acc = to_np(w4.w8a8_gemm_i32(torch.from_numpy(xq).to(dev), qd, N))
    assert np.array_equal(acc.astype(np.int64), ora.w4a8_acc_ref(xq, q, None, 128))


@pytest.mark.parametrize("M,N,K,div,parts", [(600, 1000, 2048, 32, 2), (300, 520, 1280, 64, 4)])
@pytest.mark.parametrize("depth", ["1", "0", "5"])
def test_w8a8_gemm_tail_split(M, N, K, div, parts, depth, monkeypatch):
    """The 128-row int8 GEMM (W8A8 weights) with the last tiles split over their groups
    (slot count scaled down through the tuning variables): int32 accumulators bit-exact
    and fp16 outputs within 2e-3."""
    dev = device()
    monkeypatch.setenv("W4_W4A8_SPLIT_TARGET", "1")
    monkeypatch.setenv("W4_W4A8_TAIL", "1")
    monkeypatch.setenv("W4_W4A8_BM", "128")
    monkeypatch.setenv("W4_W4A8_DEPTH", depth)
    monkeypatch.setenv("W4_W4A8_SLOTS_DIV", str(div))
    monkeypatch.setenv("W4_W4A8_TAIL_PARTS", str(parts))
    tiles = -(-M // 128) * -(-N // 256)
    rem = tiles % (512 // div)
    assert w4.w8a8_gemm_workspace_bytes(M, N, K) == 16384 + rem * parts * 128 * 256 * 4
    announce(f"w8a8 tail split M={M} N={N} K={K} tiles={tiles} parts={parts}")
    inp = synth.make_linear(M, N, K, seed=M * 7 + N, outliers=True, rms_spread=True, with_gamma=True)
    q, cs = ora.quantize_w8a8(inp.w.numpy())
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    xqd, sad = torch.from_numpy(xq).to(dev), torch.from_numpy(sa).to(dev)
    qd, csd = torch.from_numpy(ora.tile_w8a8(q)).to(dev), torch.from_numpy(cs).to(dev)
    acc = to_np(w4.w8a8_gemm_i32(xqd, qd, N))
    assert np.array_equal(acc.astype(np.int64), ora.w4a8_acc_ref(xq, q, None, 128))
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    y = to_np(w4.w8a8_gemm(xqd, sad, qd, csd, out=out)).astype(np.float64)
    assert np.all(np.isfinite(y)), "output not fully written"
    _check_fp16(y, xq, sa, q, cs)


@pytest.mark.parametrize("M,N,K", [(1, 13824, 5120), (16, 13824, 5120), (256, 13824, 5120), (4096, 13824, 5120),
                                   (4096, 5120, 13824)])
def test_w8a8_full_size_sampled(M, N, K):
    """K = 5120, N = 13824 end to end on the GPU: pack, quant_act (RMSNorm), GEMM;
    accumulators bit-exact on the oracle's xq; fp16 outputs within 2e-3.  The down shape
    (K = 13824, N = 5120) at M = 4096 takes the four-tile ring at one workgroup per CU with
    the last round's 128 tiles split in two (sampled rows and columns reach them)."""
    dev = device()
    announce(f"w8a8 full M={M} N={N} K={K}")
    inp = synth.make_linear(M, N, K, seed=0, outliers=True, rms_spread=True, with_gamma=True)
    qw, cs = w4.w8a8_pack(inp.w.to(dev))
    xq, sa = w4.w4a8_quant_act(inp.x.to(dev), inp.gamma.to(dev))
    y = w4.w8a8_gemm(xq, sa, qw, cs)
    rxq, rsa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    acc = w4.w8a8_gemm_i32(torch.from_numpy(rxq).to(dev), qw, N)
    torch.cuda.synchronize()
    ms = sample_idx(M, 48, seed=M, must=range(M - 8, M))
    ns = sample_idx(N, 256, seed=7, must=list(range(0, 32)) + list(range(N - 16, N)))
    q, rcs = ora.quantize_w8a8(inp.w.numpy()[ns])
    assert np.array_equal(ora.untile_w8a8(to_np(qw), N)[ns], q)
    racc = ora.w4a8_acc_ref(rxq[ms], q, None, 128)
    assert np.array_equal(to_np(acc)[np.ix_(ms, ns)].astype(np.int64), racc)
    _check_fp16(to_np(y)[np.ix_(ms, ns)].astype(np.float64), rxq[ms], rsa[ms], q, rcs)


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.choice([1, 2, 5, 16, 17, 33, 64, 100, 257])), int(rng.integers(1, 600)),
             128 * int(rng.integers(1, 33))) for _ in range(n)]


@pytest.mark.parametrize("M,N,K", _random_shapes(16, seed=2028))
def test_w8a8_random_shapes(M, N, K):
    dev = device()
    announce(f"w8a8 random M={M} N={N} K={K}")
    inp = synth.make_linear(M, N, K, seed=M * 17 + N + K, outliers=True, rms_spread=True, with_gamma=True)
    q, cs = ora.quantize_w8a8(inp.w.numpy())
    xq, sa, _ = ora.w4a8_quant_act_ref(inp.x.numpy(), inp.gamma.numpy())
    acc = to_np(w4.w8a8_gemm_i32(torch.from_numpy(xq).to(dev), torch.from_numpy(ora.tile_w8a8(q)).to(dev), N))
    assert np.array_equal(acc.astype(np.int64), ora.w4a8_acc_ref(xq, q, None, 128))
