"""GPU parity of the W4A16 variants: per-channel weights (group_size -1), group sizes
64 and 32, and the symmetric rule (awq_pack_sym), against the oracle.

* awq_pack / awq_pack_sym: bit-exact packed tensors, small ragged shapes, every
  combination of rule and group size, and the hand-worked rows of
  tests/golden/w4a16_variants_worked.txt;
* awq_unpack_dequant of per-channel weights: bit-exact;
* awq_gemm on oracle-packed weights through every kernel family (register-X and
  LDS-staged skinny kernels, with and without split-K, and the MFMA GEMM), within
  the normalized 2e-3 bound;
* end to end (GPU quantize + pack + GEMM) at full Llama-2-13B shapes, sampled.
"""
import numpy as np
import pytest
import torch

import oracle.ref as ora
import synth
import w4a16_gemm_amd as w4
from golden_io import read_variant_cases
from gpu_util import TOL, announce, device, normalized_error, sample_idx, to_np

pytestmark = pytest.mark.gpu

VARIANTS = [(-1, False), (128, True), (-1, True), (64, False), (32, False), (64, True), (32, True)]
VID = ["pc-asym", "g128-sym", "pc-sym", "g64-asym", "g32-asym", "g64-sym", "g32-sym"]


def _pack_gpu(w, group, sym):
    return (w4.awq_pack_sym if sym else w4.awq_pack)(w, group)


def _oracle_packed(w16, group, sym, dev):
    r = ora.awq_reference(w16, None, group, symmetric=sym)
    return r, [torch.from_numpy(np.ascontiguousarray(t)).to(dev) for t in (r["qweight"], r["scales"], r["qzeros"])]


@pytest.mark.parametrize("group,sym", VARIANTS + [(128, False)], ids=VID + ["g128-asym"])
@pytest.mark.parametrize("N,K", [(64, 128), (13, 256), (200, 384), (1000, 1024), (9, 2048)])
def test_pack_bit_exact(group, sym, N, K):
    dev = device()
    announce(f"pack group={group} sym={sym} N={N} K={K}")
    w = synth.make_linear(0, N, K, seed=N + K, outliers=True).w
    qw, sc, qz = _pack_gpu(w.to(dev), group, sym)
    torch.cuda.synchronize()
    ref = ora.awq_reference(w.numpy(), None, group, symmetric=sym)
    assert np.array_equal(to_np(qw), ref["qweight"])
    assert np.array_equal(to_np(sc).view(np.uint16), ref["scales"].view(np.uint16))
    assert np.array_equal(to_np(qz), ref["qzeros"])
    wd = w4.awq_unpack_dequant(qw, sc, qz, group)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(wd).view(np.uint16), ref["w_deq"].astype(np.float16).view(np.uint16))


def test_pack_golden_rows():
    """The hand-worked rows, quantized on the GPU."""
    dev = device()
    for c in read_variant_cases():
        announce(f"golden {c['name']}")
        w = torch.from_numpy(np.repeat(c["values"][None, :], 3, axis=0)).to(dev)
        qw, sc, qz = _pack_gpu(w, c["group"], c["rule"] == "sym")
        torch.cuda.synchronize()
        codes, scales, zeros = ora.unpack_awq(to_np(qw), to_np(sc), to_np(qz), w.shape[1])
        assert scales[0].view(np.uint16).tolist() == c["scales"].view(np.uint16).tolist(), c["name"]
        assert zeros[0].tolist() == c["zeros"], c["name"]
        for b, head in enumerate(c.get("codes_head", [])):
            assert codes[2, 128 * b:128 * b + len(head)].tolist() == head, (c["name"], b)
        for k, code in c.get("codes_at", {}).items():
            assert int(codes[2, k]) == code, (c["name"], k)


# shapes for each kernel family: register-X skinny (M <= 32, N and K <= 8192 at M <= 4),
# LDS skinny (M <= 4 with N or K > 8192; split K), MFMA GEMM (M > 32; split K for few tiles)
GEMM_SHAPES = [(1, 200, 1024), (4, 1000, 2048), (16, 520, 5120), (24, 130, 1024), (33, 96, 768), (64, 300, 640),
               (1, 200, 9216), (3, 8320, 1024), (65, 300, 640), (130, 520, 1024), (257, 1030, 2048)]


@pytest.mark.parametrize("group,sym", VARIANTS, ids=VID)
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_oracle_packed(group, sym, M, N, K):
    dev = device()
    announce(f"gemm group={group} sym={sym} M={M} N={N} K={K} ws={w4.awq_gemm_workspace_bytes(M, N, K, group)}")
    inp = synth.make_linear(M, N, K, seed=M * 5 + N + K, outliers=True, rms_spread=True)
    ref, (qw, sc, qz) = _oracle_packed(inp.w.numpy(), group, sym, dev)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    y = to_np(w4.awq_gemm(inp.x.to(dev), qw, sc, qz, group_size=group, out=out)).astype(np.float64)
    assert np.all(np.isfinite(y)), "output not fully written"
    yr = ora.linear_ref(inp.x.numpy(), ref["w_deq"])
    err = normalized_error(y, yr, np.linalg.norm(inp.x.numpy().astype(np.float64), axis=1),
                           np.linalg.norm(ref["w_deq"], axis=1))
    assert err <= TOL, err


@pytest.mark.parametrize("lds", ["0", "1"])
@pytest.mark.parametrize("M,N,K", [(1, 520, 5120), (4, 200, 13824), (16, 130, 2048)])
def test_gemm_per_channel_both_skinny_kernels(lds, M, N, K, monkeypatch):
    """Per-channel weights through the register-X and the LDS skinny kernel alike."""
    dev = device()
    monkeypatch.setenv("W4_SKINNY_LDS", lds)
    announce(f"per-channel skinny lds={lds} M={M} N={N} K={K}")
    inp = synth.make_linear(M, N, K, seed=M + N, outliers=True)
    ref, (qw, sc, qz) = _oracle_packed(inp.w.numpy(), -1, False, dev)
    y = to_np(w4.awq_gemm(inp.x.to(dev), qw, sc, qz, group_size=-1)).astype(np.float64)
    yr = ora.linear_ref(inp.x.numpy(), ref["w_deq"])
    err = normalized_error(y, yr, np.linalg.norm(inp.x.numpy().astype(np.float64), axis=1),
                           np.linalg.norm(ref["w_deq"], axis=1))
    assert err <= TOL, err


@pytest.mark.parametrize("group,sym", VARIANTS, ids=VID)
@pytest.mark.parametrize("M,N,K", [(1, 27648, 5120), (16, 5120, 13824), (4096, 5120, 5120)])
def test_full_size_end_to_end_sampled(group, sym, M, N, K):
    """GPU quantize + pack + GEMM at full Llama-2-13B shapes; sampled outputs against
    the oracle's chain on the sampled rows and columns."""
    dev = device()
    announce(f"variants full size group={group} sym={sym} M={M} N={N} K={K}")
    w = synth.make_linear(0, N, K, seed=3, outliers=True).w
    qw, sc, qz = _pack_gpu(w.to(dev), group, sym)
    x = synth.make_activations(M, K, seed=M, rms_spread=True)
    y = w4.awq_gemm(x.to(dev), qw, sc, qz, group_size=group)
    torch.cuda.synchronize()
    ms = sample_idx(M, 32, seed=M)
    ns = sample_idx(N, 256, seed=N + M, must=range(0, 32))
    ref = ora.awq_reference(w.numpy()[ns], x.numpy()[ms], group, symmetric=sym)
    yg = to_np(y)[np.ix_(ms, ns)].astype(np.float64)
    err = normalized_error(yg, ref["y"], np.linalg.norm(x.numpy()[ms].astype(np.float64), axis=1),
                           np.linalg.norm(ref["w_deq"], axis=1))
    assert err <= TOL, err


@pytest.mark.parametrize("group", [32, 64, -1])
def test_identity_probe_bit_exact(group):
    """X rows are unit vectors e_k (k on both sides of group boundaries): Y[m, n] is the
    fp16 dequantized weight bit for bit, so every lane reads the scale and zero point of
    its own group."""
    dev = device()
    N, K, M = 320, 1024, 96
    announce(f"identity probe group={group}")
    w = synth.make_linear(0, N, K, seed=19, outliers=True).w.numpy()
    ref, (qw, sc, qz) = _oracle_packed(w, group, False, dev)
    ks = sample_idx(K, M, seed=group + 5, must=(0, 31, 32, 63, 64, 95, 96, 127, 128, 1023))[:M]
    x = np.zeros((M, K), np.float16)
    x[np.arange(len(ks)), ks] = 1
    y = to_np(w4.awq_gemm(torch.from_numpy(x).to(dev), qw, sc, qz, group_size=group))
    expect = ref["w_deq"][:, ks].T.astype(np.float16)
    assert np.array_equal(y[:len(ks)].view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("tiles", ["1", "2", "4", "8"])
@pytest.mark.parametrize("M,N,K", [(1, 200, 1024), (16, 520, 5120), (5, 130, 13824), (24, 96, 768)])
def test_dequantizing_skinny_every_tile_width(group, tiles, M, N, K, monkeypatch):
    """Group sizes 64 and 32 at M <= 32 take the dequantizing register-X kernel: each tile
    width (forced through its tuning variable), split K, ragged N."""
    dev = device()
    monkeypatch.setenv("W4_SKINNY_TILES", tiles)
    announce(f"dequantizing skinny group={group} tiles={tiles} M={M} N={N} K={K}")
    inp = synth.make_linear(M, N, K, seed=M + N + group, outliers=True, rms_spread=True)
    ref, (qw, sc, qz) = _oracle_packed(inp.w.numpy(), group, False, dev)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    y = to_np(w4.awq_gemm(inp.x.to(dev), qw, sc, qz, group_size=group, out=out)).astype(np.float64)
    assert np.all(np.isfinite(y)), "output not fully written"
    yr = ora.linear_ref(inp.x.numpy(), ref["w_deq"])
    err = normalized_error(y, yr, np.linalg.norm(inp.x.numpy().astype(np.float64), axis=1),
                           np.linalg.norm(ref["w_deq"], axis=1))
    assert err <= TOL, err
