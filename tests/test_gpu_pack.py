"""GPU parity: weight quantization and packing are bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle.ref as ora
import synth
import w4a16_gemm_amd as w4
from golden_io import read_cases
from gpu_util import announce, device, sample_idx, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,outliers", [
    (64, 128, False), (200, 384, True), (1000, 1024, True), (13, 256, False), (8, 128, True),
])
def test_awq_pack_bit_exact_small(N, K, outliers):
    dev = device()
    announce(f"awq_pack N={N} K={K}")
    w = synth.make_linear(0, N, K, seed=N + K, outliers=outliers).w
    qw, sc, qz = w4.awq_pack(w.to(dev))
    torch.cuda.synchronize()
    codes, scales, zeros = ora.quantize_asym(w.numpy(), 128)
    rqw, rsc, rqz = ora.pack_awq(codes, scales, zeros)
    assert np.array_equal(to_np(qw), rqw)
    assert np.array_equal(to_np(sc).view(np.uint16), rsc.view(np.uint16))
    assert np.array_equal(to_np(qz), rqz)
    # the exported dequantized weights: fp16 of (q - z) * s, one rounding
    wd = w4.awq_unpack_dequant(qw, sc, qz)
    torch.cuda.synchronize()
    ref = ora.dequant_awq(rqw, rsc, rqz, K, 128).astype(np.float16)
    assert np.array_equal(to_np(wd).view(np.uint16), ref.view(np.uint16))


def test_awq_pack_golden_groups():
    """The hand-worked groups of tests/golden/asym_g128_worked.txt, on the GPU."""
    dev = device()
    cases = read_cases("asym_g128_worked.txt")
    w = (np.random.default_rng(5).standard_normal((len(cases), 256)) * 0.02).astype(np.float16)
    for i, c in enumerate(cases):
        w[i, 128:] = c["values"]
    qw, sc, qz = w4.awq_pack(torch.from_numpy(w).to(dev))
    torch.cuda.synchronize()
    codes, scales_nk, zeros_nk = ora.unpack_awq(to_np(qw), to_np(sc), to_np(qz), 256)
    for i, c in enumerate(cases):
        assert scales_nk[i, 1].view(np.uint16) == c["scale"].view(np.uint16), c["name"]
        assert int(zeros_nk[i, 1]) == c["zero"], c["name"]
        for j, v in enumerate(c["values"]):
            hx = format(int(v.view(np.uint16)), "04X")
            assert int(codes[i, 128 + j]) == c["code"][hx], (c["name"], hx)


@pytest.mark.parametrize("shape", [(4096, 4096), (15360, 5120), (5120, 5120), (27648, 5120), (5120, 13824),
                                   (13824, 5120)])
def test_awq_pack_bit_exact_full_shapes(shape):
    """Full Llama-2-13B weight shapes: sampled rows are bit-exact."""
    dev = device()
    N, K = shape
    announce(f"awq_pack full N={N} K={K}")
    w = synth.make_linear(0, N, K, seed=0, outliers=(N, K) != (4096, 4096)).w
    qw, sc, qz = w4.awq_pack(w.to(dev))
    torch.cuda.synchronize()
    rows = sample_idx(N, 192, seed=N, must=range(0, 16))
    codes, scales, zeros = ora.quantize_asym(w.numpy()[rows], 128)
    rqw, _, _ = ora.pack_awq(codes, scales, zeros)
    assert np.array_equal(ora.untile_words(to_np(qw), N)[rows], ora.untile_words(rqw, len(rows)))
    assert np.array_equal(to_np(sc)[:, rows].view(np.uint16), np.ascontiguousarray(scales.T).view(np.uint16))
    g_codes, _, g_zeros = ora.unpack_awq(to_np(qw), to_np(sc), to_np(qz), K)
    assert np.array_equal(g_zeros[rows], zeros)


@pytest.mark.parametrize("group", [-1, 128])
@pytest.mark.parametrize("N,K", [(64, 256), (200, 1024), (13824, 5120)])
def test_w4a8_pack_bit_exact(group, N, K):
    dev = device()
    announce(f"w4a8_pack N={N} K={K} group={group}")
    w = synth.make_linear(0, N, K, seed=3, outliers=True).w
    qw, gs, cs = w4.w4a8_pack(w.to(dev), group)
    torch.cuda.synchronize()
    rows = sample_idx(N, 256, seed=1) if N > 256 else np.arange(N)
    q, rcs, rgs = ora.quantize_w4a8(w.numpy()[rows], group)
    rqw, rcs2, rgs_gn = ora.pack_w4a8(q, rcs, rgs)
    assert np.array_equal(ora.untile_words(to_np(qw), N)[rows], ora.untile_words(rqw, len(rows)))
    if N <= 256:
        assert np.array_equal(to_np(qw), rqw)  # whole tiled array, padding rows included
    assert np.array_equal(to_np(cs)[rows].view(np.uint16), rcs2.view(np.uint16))
    if group == -1:
        assert gs is None
    else:
        assert np.array_equal(to_np(gs)[:, rows], rgs_gn)


def test_w4a8_pack_golden_rows():
    dev = device()
    for c in read_cases("w4a8_worked.txt"):
        # rows shorter than one 128-group are zero-padded (padding leaves max|w| unchanged)
        K = max(128, c["values"].size)
        row = np.zeros(K, np.float16)
        row[:c["values"].size] = c["values"]
        w = np.tile(row[None, :], (8, 1))
        qw, gs, cs = w4.w4a8_pack(torch.from_numpy(w).to(dev), c["group"])
        torch.cuda.synchronize()
        q = ora.unpack_w4a8(to_np(qw), 8, K)
        assert to_np(cs)[0].view(np.uint16) == c["cscale"].view(np.uint16)
        if c["group"] == -1:
            assert q[0, :len(c["q"])].tolist() == c["q"]
        else:
            assert to_np(gs)[:, 0].tolist() == c["gscale"]
            for g, head in enumerate(c["q_head"]):
                assert q[0, g * 128:g * 128 + len(head)].tolist() == head


@pytest.mark.parametrize("R,C", [(1, 8), (37, 131), (300, 1000), (5, 3), (64, 640)])
def test_pack_codes_bit_exact(R, C):
    """w4_pack_codes: plain row-major nibble packing, against the oracle's packer (ragged
    C: trailing nibbles 0), codes spanning 0..15."""
    dev = device()
    announce(f"w4_pack_codes R={R} C={C}")
    codes = synth.uniform_ints((R, C), 0, 15, seed=R * 31 + C).numpy().astype(np.uint8)
    codes[0, 0] = 15
    out = w4.w4_pack_codes(torch.from_numpy(codes).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), ora.pack_nibbles(codes))
