"""GPU: awq_gemm_noalloc (the entry point for callers that cannot allocate) gives the
outputs of awq_gemm bit for bit, through the C ABI, on calls in a row that share the
static workspace -- a large prefill call with a tail split, then smaller ones that split
K -- and refuses a shape whose workspace exceeds the static array before any launch."""
import pytest
import torch

import synth
import w4a16_gemm_amd as w4
from gpu_util import announce, device

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def test_noalloc_matches_awq_gemm_on_consecutive_calls():
    dev = device()
    lib = w4.load()
    for M, N, K in [(4096, 5120, 5120), (64, 5120, 5120), (16, 5120, 13824), (1, 256, 5120)]:
        announce(f"awq_gemm_noalloc M={M} N={N} K={K}")
        need = lib.awq_gemm_workspace_bytes(M, N, K, 128)
        assert 0 < need <= SCRATCH
        inp = synth.make_linear(M, N, K, seed=M + N, outliers=True, rms_spread=True)
        qw, sc, qz = w4.awq_pack(inp.w.to(dev))
        x = inp.x.to(dev)
        ref = w4.awq_gemm(x, qw, sc, qz)
        out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        w4.awq_gemm_noalloc(x, qw, sc, qz, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        # the same call again (the workspace's counters were left at zero)
        out.fill_(float("nan"))
        w4.awq_gemm_noalloc(x, qw, sc, qz, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_noalloc_refuses_workspace_above_the_static_array(monkeypatch):
    dev = device()
    # 768 tiles on 512 slots: the last 256 split in two (forced; the default plan splits a
    # last round only up to a quarter of the slots) need 64 MiB + 16 KiB of partials
    monkeypatch.setenv("W4_GEMM_TAIL", "1")
    M, N, K = 4096, 6144, 5120
    announce(f"awq_gemm_noalloc refusal M={M} N={N} K={K}")
    assert w4.load().awq_gemm_workspace_bytes(M, N, K, 128) > SCRATCH
    x = torch.zeros((M, K), dtype=torch.float16, device=dev)
    qw = torch.zeros(w4.qweight_shape(N, K), dtype=torch.int32, device=dev)
    sc = torch.zeros((K // 128, N), dtype=torch.float16, device=dev)
    qz = torch.zeros((K // 128, (N + 7) // 8), dtype=torch.int32, device=dev)
    out = torch.zeros((M, N), dtype=torch.float16, device=dev)
    with pytest.raises(w4.W4Error, match="static"):
        w4.awq_gemm_noalloc(x, qw, sc, qz, out)
    torch.cuda.synchronize()
    assert not out.any()
