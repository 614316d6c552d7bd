"""GPU: the entry points under stream capture.  Bound calls (pre-marshalled arguments,
workspace allocated and zeroed at bind time) are captured into one HIP graph on a side
stream and replayed several times, with eager launches of the same calls and output
poisoning between replays; every replay must reproduce the eager outputs bit for bit
(the kernels are deterministic, and the split-K arrival counters return to zero at the
end of every call, so a replay needs no memset)."""
import pytest
import torch

import synth
import w4a16_gemm_amd as w4
from gpu_util import announce, device

pytestmark = pytest.mark.gpu


def _bound_calls(dev):
    calls, outs = [], []
    # W4A16: a split-K skinny shape (narrow N), the LDS skinny kernel, the MFMA GEMM
    for (M, N, K) in ((4, 256, 5120), (1, 9000, 1024), (16, 520, 5120), (96, 256, 1024)):
        inp = synth.make_linear(M, N, K, seed=M + N, outliers=True)
        qw, sc, qz = w4.awq_pack(inp.w.to(dev))
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        calls.append(w4.bind_awq_gemm(inp.x.to(dev), qw, sc, qz, y))
        outs.append(y)
    # W4A8 chain at M = 16 (split-K skinny int8 kernel) and W8A8
    inp = synth.make_linear(16, 1000, 2048, seed=3, outliers=True, rms_spread=True, with_gamma=True)
    xq = torch.empty((16, 2048), dtype=torch.int8, device=dev)
    sa = torch.empty((16,), dtype=torch.float32, device=dev)
    calls.append(w4.bind_w4a8_quant_act(inp.x.to(dev), inp.gamma.to(dev), xq, sa))
    outs += [xq, sa]
    qw, gs, cs = w4.w4a8_pack(inp.w.to(dev), 128)
    y8 = torch.empty((16, 1000), dtype=torch.float16, device=dev)
    calls.append(w4.bind_w4a8_gemm(xq, sa, qw, gs, cs, y8, 128))
    outs.append(y8)
    q8, c8 = w4.w8a8_pack(inp.w.to(dev))
    y88 = torch.empty((16, 1000), dtype=torch.float16, device=dev)
    calls.append(w4.bind_w8a8_gemm(xq, sa, q8, c8, y88))
    outs.append(y88)
    gu = synth.make_activations(8, 2 * 1024, seed=4, rms_spread=True).to(dev)
    xs = torch.empty((8, 1024), dtype=torch.int8, device=dev)
    ss = torch.empty((8,), dtype=torch.float32, device=dev)
    calls.append(w4.bind_w4a8_silu_mul_quant(gu, xs, ss))
    outs += [xs, ss]
    return calls, outs


def _same(a, b):
    if a.dtype in (torch.int8, torch.uint8):
        return torch.equal(a, b)
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _poison(outs):
    for t in outs:
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-1)


def test_graph_replays_match_eager():
    dev = device()
    announce("graph capture and replay")
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        calls, outs = _bound_calls(dev)  # binds to the side stream; workspaces zeroed here
        for c in calls:
            c()
    side.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in calls:
            c()
    for rep in range(4):
        with torch.cuda.stream(side):
            _poison(outs)
            graph.replay()
        side.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same(a, b), f"replay {rep}, output {i}"
        # eager launches of the same calls between replays (counters must stay consistent)
        with torch.cuda.stream(side):
            _poison(outs)
            for c in calls:
                c()
        side.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same(a, b), f"eager after replay {rep}, output {i}"
