"""GPU: plain-layout weights imported through the C-ABI (awq_import_plain,
w4a8_import_plain) equal the oracle's packed layout bit for bit, and the imported
weights drive the GEMMs exactly as the library's own packer does.

The plain layouts are the Triton AWQ weight format printed on "Implement AWQ
quantization support for LLaMA" (codes packed 8 per word along K, per-group scales,
zero points packed along the group axis), per output channel ("rows") or K-major as
printed ("cols")."""
import numpy as np
import pytest
import torch

import synth
import w4a16_gemm_amd as w4
from oracle import ref as ora
from gpu_util import announce, device, to_np

pytestmark = pytest.mark.gpu


def _plain_awq(codes, scales, zeros, layout):
    """Oracle codes / scales / zeros [N, .] -> the plain layout's three arrays."""
    words = ora.pack_nibbles(codes)
    zw = ora.pack_nibbles(zeros)
    if layout == "rows":
        return words, np.ascontiguousarray(scales), zw
    return np.ascontiguousarray(words.T), np.ascontiguousarray(scales.T), np.ascontiguousarray(zw.T)


@pytest.mark.parametrize("layout", ["rows", "cols"])
@pytest.mark.parametrize("group", [128, 64, 32, -1])
@pytest.mark.parametrize("N,K", [(40, 384), (16, 128), (77, 1152)])
def test_awq_import_matches_oracle_packing(N, K, group, layout):
    dev = device()
    announce(f"awq_import_plain N={N} K={K} g={group} {layout}")
    w = synth.make_linear(1, N, K, seed=N + K + group, outliers=True).w
    codes, s, z = ora.quantize_asym(w.numpy(), group)
    qw_p, s_p, z_p = _plain_awq(codes, s, z, layout)
    qw, sc, qz = w4.awq_import_plain(torch.from_numpy(qw_p).to(dev), torch.from_numpy(s_p).to(dev),
                                     torch.from_numpy(z_p).to(dev), group, layout)
    torch.cuda.synchronize()
    rq, rs, rz = ora.pack_awq(codes, s, z)
    assert np.array_equal(to_np(qw), rq)
    assert np.array_equal(to_np(sc).view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(to_np(qz), rz)
    # the library's own packer from the fp16 weights gives the same arrays
    pq, ps, pz = w4.awq_pack(w.to(dev), group)
    torch.cuda.synchronize()
    assert torch.equal(pq, qw) and torch.equal(ps.view(torch.int16), sc.view(torch.int16)) and torch.equal(pz, qz)


@pytest.mark.parametrize("layout", ["rows", "cols"])
@pytest.mark.parametrize("group", [128, -1])
@pytest.mark.parametrize("N,K", [(40, 384), (300, 1024)])
def test_w4a8_import_matches_oracle_packing(N, K, group, layout):
    dev = device()
    announce(f"w4a8_import_plain N={N} K={K} g={group} {layout}")
    w = synth.make_linear(1, N, K, seed=N + K + 7, outliers=True).w
    q, cs, gs = ora.quantize_w4a8(w.numpy(), group)
    words = ora.pack_nibbles(q.astype(np.int64) + 8)
    gsp = None if gs is None else gs
    if layout == "cols":
        words = np.ascontiguousarray(words.T)
        gsp = None if gs is None else np.ascontiguousarray(gs.T)
    qw, g2 = w4.w4a8_import_plain(torch.from_numpy(words).to(dev),
                                  None if gsp is None else torch.from_numpy(gsp).to(dev), group, layout)
    torch.cuda.synchronize()
    rq, _, rg = ora.pack_w4a8(q, cs, gs)
    assert np.array_equal(to_np(qw), rq)  # includes the padding rows (q = 0, nibble 8)
    if group == -1:
        assert g2 is None
    else:
        assert np.array_equal(to_np(g2), rg)
    pq, pg, _ = w4.w4a8_pack(w.to(dev), group)
    torch.cuda.synchronize()
    assert torch.equal(pq, qw) and (group == -1 or torch.equal(pg, g2))


@pytest.mark.parametrize("layout", ["rows", "cols"])
def test_full_size_codes_packed_on_gpu_then_imported(layout):
    """Down projection 13824 -> 5120: oracle codes / zero points packed into plain words
    by the GPU packer (w4_pack_codes), imported, and used by awq_gemm give the arrays and
    the outputs of awq_pack -> awq_gemm bit for bit."""
    dev = device()
    N, K, M = 5120, 13824, 4
    announce(f"import chain N={N} K={K} {layout}")
    inp = synth.make_linear(M, N, K, seed=11, outliers=True)
    codes, s, z = ora.quantize_asym(inp.w.numpy(), 128)
    words = w4.w4_pack_codes(torch.from_numpy(codes).to(dev))
    zw = w4.w4_pack_codes(torch.from_numpy(z).to(dev))
    sp = torch.from_numpy(s).to(dev)
    if layout == "cols":
        words, zw, sp = words.t().contiguous(), zw.t().contiguous(), sp.t().contiguous()
    qw, sc, qz = w4.awq_import_plain(words, sp, zw, 128, layout)
    pq, ps, pz = w4.awq_pack(inp.w.to(dev), 128)
    torch.cuda.synchronize()
    assert torch.equal(pq, qw) and torch.equal(ps.view(torch.int16), sc.view(torch.int16)) and torch.equal(pz, qz)
    x = inp.x.to(dev)
    y_imp = w4.awq_gemm(x, qw, sc, qz)
    y_own = w4.awq_gemm(x, pq, ps, pz)
    torch.cuda.synchronize()
    assert torch.equal(y_imp.view(torch.int16), y_own.view(torch.int16))
