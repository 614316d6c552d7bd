#!/usr/bin/env python3
"""Throughput of the W4A16-g128 linear layer on one MI355X.

Default workload: the Llama-2-13B decode projection set -- fused QKV (K=5120,
N=15360), O (5120, 5120), fused gate+up (5120, 27648) and down (13824, 5120) -- at
M in {1, 4, 16} tokens.  One step = the 12 awq_gemm calls (every projection at every
M).  Inputs are seeded synthetic tensors (weights ~N(0, 0.02) with 1% outlier input
channels x10, activations ~N(0, 1)), quantized and packed on the GPU before timing;
everything is resident in HBM when the timed region starts.  To keep the 256 MB
Infinity Cache from serving weights, R copies of every packed weight set are rotated
so that a weight set is re-read only after ~R x 165 MB of other weights.

value = algorithmic bytes of all timed calls / wall time of the timed region (GB/s).
Algorithmic bytes of one call: N*K/2 (codes) + 2*N*K/G (scales) + N*K/(2G) (zeros)
+ 2*M*K (X) + 2*M*N (Y).

The JSON line also carries
  roofline      the dominant kernel (the skinny M<=16 kernel: every decode call) from
                per-launch HIP events recorded between the launches of the timed region
  cpu_baseline  the CPU oracle (numpy dequant + fp64 matmul) on one decode step
  detail        the other workloads (single M=8 GEMM, the batch crossover sweep, the
                M=4096 prefill GEMMs in TFLOP/s, the W4A8 stage), timed separately
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2**20  # Infinity Cache (last-level, in front of HBM)
F16_PEAK_TFLOPS = 2516.6
I8_PEAK_TOPS = 5033.2
G = 128


def awq_bytes(M, N, K):
    return N * K / 2 + 2 * N * (K // G) + N * (K // G) / 2 + 2 * M * K + 2 * M * N


def w4a8_bytes(M, N, K, two_level):
    return N * K / 2 + 2 * N + (N * (K // G) if two_level else 0) + M * K + 4 * M + 2 * M * N


def profiled_traffic(key):
    """HBM bytes per launch of a kernel as measured by the committed counter runs
    (FETCH_SIZE and WRITE_SIZE, calibrated on a plain copy), or None when the kernel's
    sources have changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[key]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec["source_hash"]:
        return None
    return rec["hbm_bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4, help="copies of each packed weight set")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--detail-iters", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "w4a8", "copy", "micro", "small", "midm"],
                    help="decode (default, the reported metric); prefill / w4a8 (the int8 path) / copy run one kernel family "
                         "alone (for profiling); copy is a plain device copy of known size that calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters; micro measures the ceilings (HBM read stream "
                         "at the decode weight sizes and 1 GiB, fp16 / int8 MFMA loops); small runs the single "
                         "M=8 GEMM and the O projection at M=1,4,16; midm the crossover shapes M=64,128,256")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def rotated_awq(qw, sc, qz, r):
    """Copy r of a packed W4A16 weight: the same matrix with its rows (output channels)
    rolled by 112 r (7 r tiles of 16), a distinct buffer in HBM for cache rotation."""
    import torch
    return (torch.roll(qw, 7 * r, 0).contiguous(), torch.roll(sc, 112 * r, 1).contiguous(),
            torch.roll(qz, 14 * r, 1).contiguous())


def rotated_w4a8(qw, gs, cs, r):
    import torch
    return (torch.roll(qw, 7 * r, 0).contiguous(), None if gs is None else torch.roll(gs, 112 * r, 1).contiguous(),
            torch.roll(cs, 112 * r, 0).contiguous())


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 (sharding the layer over "
                          "several GPUs is not implemented)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w4a16_gemm_amd as w4

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w4.load()
    if args.workload == "micro":
        print(json.dumps(micro(args, dev, torch, w4)), flush=True)
        return
    if args.workload != "decode":
        print(json.dumps(single_workload(args, dev, torch, np, synth, w4)), flush=True)
        return

    # ---------------------------------------------------------------- inputs
    log("generating inputs")
    host = {}
    packed = {}
    for name, (K, N) in synth.LLAMA2_13B.items():
        inp = synth.make_linear(16, N, K, seed=0, outliers=True)
        host[name] = inp
        qw, sc, qz = w4.awq_pack(inp.w.to(dev))
        packed[name] = [rotated_awq(qw, sc, qz, r) for r in range(args.rotate)]
        del qw, sc, qz
    torch.cuda.synchronize()

    Ms = (1, 4, 16)
    names = list(synth.LLAMA2_13B)
    xs = {(name, M): host[name].x[:M].contiguous().to(dev) for name in names for M in Ms}
    ys = {(name, M): torch.empty((M, synth.LLAMA2_13B[name][1]), dtype=torch.float16, device=dev)
          for name in names for M in Ms}
    # calls[i] for round j: projections in order, M fixed per round, weight copy j % R
    rounds = []
    for j in range(len(Ms) * args.rotate):
        M = Ms[j % len(Ms)]
        r = j % args.rotate
        rounds.append([(name, M, w4.bind_awq_gemm(xs[(name, M)], *packed[name][r], ys[(name, M)]))
                       for name in names])
    per_step = len(Ms) * len(names)
    byts = {(name, M): awq_bytes(M, synth.LLAMA2_13B[name][1], synth.LLAMA2_13B[name][0])
            for name in names for M in Ms}
    step_bytes = sum(byts.values())

    def calls_for_step(s):
        out = []
        for j in range(len(Ms)):
            out += rounds[(s * len(Ms) + j) % len(rounds)]
        return out

    # --------------------------------------------------------------- warmup
    log(f"warmup {args.warmup} steps")
    for s in range(args.warmup):
        for (_, _, fn) in calls_for_step(s):
            fn()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    # The timed region is bracketed by two HIP events on the launch stream and holds
    # nothing but the launches.  Every launch is the same kernel family (the skinny
    # M <= 16 kernel), so its average launch duration is the region time / launches.
    stream = torch.cuda.current_stream(dev)
    n_launch = per_step * args.steps
    plan = [calls_for_step(args.warmup + s) for s in range(args.steps)]
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"timed {args.steps} steps x {per_step} launches")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for s in range(args.steps):
        for (_, _, fn) in plan[s]:
            fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev0.elapsed_time(ev1)
    gbs = step_bytes * args.steps / (total_ms * 1e-3) / 1e9
    avg_us = total_ms * 1e3 / n_launch
    achieved = gbs
    log(f"timed region {total_ms:.3f} ms (host wall {wall * 1e3:.1f} ms): {gbs:.1f} GB/s")
    # per-shape breakdown (outside the timed region): back-to-back launches of one shape,
    # rotating enough weight copies that one copy's reuse distance exceeds twice the
    # 256 MB Infinity Cache (the small shapes would otherwise be served from it)
    shape_detail = {}
    for name in names:
        wbytes = sum(t.numel() * t.element_size() for t in packed[name][0])
        ncopy = max(args.rotate, -(-2 * MALL_BYTES // wbytes))
        copies = packed[name] + [rotated_awq(*packed[name][0], r) for r in range(args.rotate, ncopy)]
        for M in Ms:
            calls = [w4.bind_awq_gemm(xs[(name, M)], *c, ys[(name, M)]) for c in copies]
            t = _time_calls(torch, calls, max(8 * args.rotate, 2 * ncopy))
            b = byts[(name, M)]
            shape_detail[f"{name}_M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1),
                                            "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 3)}
        del copies, calls

    copy_gbs = _copy_bandwidth(torch, dev)
    log(f"plain device copy: {copy_gbs:.0f} GB/s (read + write)")
    # measured ceiling of the same step: a read-only stream kernel reading, launch for
    # launch, the algorithmic bytes of each of the step's calls from buffers rotated over
    # 1 GiB (best of a few grid shapes); its per-launch average is what the skinny kernel
    # could reach if it did nothing but stream its bytes
    step_sizes = [byts[(name, M)] for M in Ms for name in names]
    ceil = _read_ceiling(torch, w4, dev, step_sizes, args.steps)
    log(f"read-stream ceiling of the step: {ceil['GBps']:.0f} GB/s ({ceil['config']})")
    result = {
        "metric": "W4A16-g128 GEMM GB/s (M<=16) & TFLOP/s (M>=256) vs roofline, 13B shapes",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; W~N(0,0.02) with 1% outlier input channels x10, X~N(0,1))",
        "config": {"workload": "Llama-2-13B decode projection set: QKV 5120x15360, O 5120x5120, "
                               "gate+up 5120x27648, down 13824x5120 at M in {1,4,16}; g128 asymmetric uint4",
                   "launches_per_step": per_step, "weight_copies_rotated": args.rotate,
                   "bytes_per_step": int(step_bytes)},
        "roofline": {"bound": "hbm", "kernel": "skinny_kernel (awq_gemm, M<=16)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(avg_us, 3),
                     "algorithmic_bytes_per_launch": int(step_bytes / per_step),
                     "traffic": profiled_traffic("skinny_decode_13b"),
                     # measured ceiling: a read-only HBM stream kernel over the same byte counts,
                     # launch for launch (ceilings.hip; profiles/ceilings.md)
                     "measured_peak": round(ceil["GBps"], 1),
                     "frac_of_measured": round(achieved / ceil["GBps"], 4),
                     "measured_peak_kernel": "read_stream_kernel " + ceil["config"],
                     # context: what a plain 1 GiB device copy (torch) reaches on this part
                     "copy_GBps": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4)},
        "per_shape": shape_detail,
    }

    if not args.no_detail:
        result["detail"] = detail(args, dev, torch, np, synth, w4, host, packed)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, synth, host)
    print(json.dumps(result), flush=True)


def single_workload(args, dev, torch, np, synth, w4):
    """One kernel family alone, for profiling: K timed iterations after W warmups."""
    res = {"workload": args.workload, "steps": args.steps, "warmup": args.warmup}
    if args.workload == "copy":
        n = 512 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        calls = [lambda: b.copy_(a)]
        res["bytes_read_per_call"] = n
        res["bytes_written_per_call"] = n
    elif args.workload == "prefill":
        calls = []
        for (K, N) in ((5120, 27648), (5120, 5120), (13824, 5120)):
            inp = synth.make_linear(0, N, K, seed=0, outliers=True)
            qw, sc, qz = w4.awq_pack(inp.w.to(dev))
            x = synth.make_activations(4096, K, seed=4096, rms_spread=True).to(dev)
            y = torch.empty((4096, N), dtype=torch.float16, device=dev)
            calls.append(w4.bind_awq_gemm(x, qw, sc, qz, y))
        res["flops_per_round"] = sum(2.0 * 4096 * N * K for (K, N) in ((5120, 27648), (5120, 5120), (13824, 5120)))
    elif args.workload == "small":
        # the single M = 8 GEMM (4096 x 4096) and the O projection (5120 x 5120) at
        # M = 1, 4, 16, each over enough rotated weight copies to stream from HBM
        calls = []
        for (M, K, N) in ((8, 4096, 4096), (1, 5120, 5120), (4, 5120, 5120), (16, 5120, 5120)):
            inp = synth.make_linear(M, N, K, seed=0, outliers=(N != 4096))
            qw, sc, qz = w4.awq_pack(inp.w.to(dev))
            x = inp.x.to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            nc = -(-2 * MALL_BYTES // int(awq_bytes(0, N, K)))
            calls += [w4.bind_awq_gemm(x, *rotated_awq(qw, sc, qz, r), y) for r in range(nc)]
        res["launches_per_round"] = len(calls)
    elif args.workload == "midm":
        # the crossover shape K = 5120, N = 13824 at M = 64, 128, 256 (16 rotated copies)
        calls = []
        inp = synth.make_linear(256, 13824, 5120, seed=0, outliers=True)
        qw, sc, qz = w4.awq_pack(inp.w.to(dev))
        copies = [rotated_awq(qw, sc, qz, r) for r in range(16)]
        for M in (64, 128, 256):
            x = inp.x[:M].contiguous().to(dev)
            y = torch.empty((M, 13824), dtype=torch.float16, device=dev)
            calls += [w4.bind_awq_gemm(x, *c, y) for c in copies]
        res["launches_per_round"] = len(calls)
    else:  # the int8 path at M = 4096: quant_act, W4A8 (both weight variants), W8A8, silu_mul_quant
        inp = synth.make_linear(4096, 13824, 5120, seed=0, outliers=True, rms_spread=True, with_gamma=True)
        x = inp.x.to(dev)
        g = inp.gamma.to(dev)
        xq = torch.empty((4096, 5120), dtype=torch.int8, device=dev)
        sa = torch.empty((4096,), dtype=torch.float32, device=dev)
        calls = [w4.bind_w4a8_quant_act(x, g, xq, sa)]
        for group in (-1, 128):
            qw, gs, cs = w4.w4a8_pack(inp.w.to(dev), group)
            y = torch.empty((4096, 13824), dtype=torch.float16, device=dev)
            calls.append(w4.bind_w4a8_gemm(xq, sa, qw, gs, cs, y, group))
        qw8, cs8 = w4.w8a8_pack(inp.w.to(dev))
        y8 = torch.empty((4096, 13824), dtype=torch.float16, device=dev)
        calls.append(w4.bind_w8a8_gemm(xq, sa, qw8, cs8, y8))
        gu = synth.make_activations(4096, 2 * 13824, seed=5, rms_spread=True).to(dev)
        xq2 = torch.empty((4096, 13824), dtype=torch.int8, device=dev)
        sa2 = torch.empty((4096,), dtype=torch.float32, device=dev)
        calls.append(w4.bind_w4a8_silu_mul_quant(gu, xq2, sa2))
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(args.steps):
        for c in calls:
            c()
    a1.record()
    torch.cuda.synchronize()
    res["ms_per_round"] = a0.elapsed_time(a1) / args.steps
    return res


READ_CONFIGS = ((256, 8), (512, 4), (512, 8), (1024, 4), (2048, 4), (1024, 8), (2048, 8), (4096, 4))


def _read_ceiling(torch, w4, dev, sizes, steps, pool_bytes=1 << 30):
    """Read-only stream ceiling of a sequence of launches: one w4_ceiling_read launch per
    entry of `sizes` (bytes), each over a fresh region of a 1 GiB pool (consecutive
    launches read consecutive regions, so no byte is re-read within 1 GiB: beyond the
    256 MB Infinity Cache), the sequence repeated `steps` times.  Best over a few grid
    shapes.  Returns GB/s = bytes / event time and the average launch time."""
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pool.fill_(0x5A)
    sizes = [int(-(-b // 256) * 256) for b in sizes]
    best = None
    for blocks, unroll in READ_CONFIGS:
        calls, off = [], 0
        for b in sizes * max(1, min(steps, 64)):
            if off + b > pool_bytes:
                off = 0
            calls.append(w4.bind_ceiling_read(pool[off:off + b], b, blocks, unroll))
            off += b
        for c in calls[: len(sizes)]:
            c()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for c in calls:
            c()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        nbytes = float(sum(sizes)) * (len(calls) // len(sizes))
        r = {"GBps": nbytes / t / 1e9, "avg_launch_us": t / len(calls) * 1e6,
             "config": f"blocks={blocks} unroll={unroll}"}
        if best is None or r["GBps"] > best["GBps"]:
            best = r
    del pool
    return best


def micro(args, dev, torch, w4):
    """Measured ceilings: the HBM read stream at each decode call's weight size, the
    single M=8 GEMM's size and 1 GiB (every grid shape of READ_CONFIGS), and fp16 / int8
    MFMA issue loops on constant and random operands (a few occupancies)."""
    import synth
    res = {"workload": "micro", "read_stream": {}, "mfma": {}}
    sizes = {"single_m8_4096": awq_bytes(8, 4096, 4096)}
    for name, (K, N) in synth.LLAMA2_13B.items():
        sizes[f"{name}_M1"] = awq_bytes(1, N, K)
    sizes["1GiB"] = float(1 << 30)
    pool = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    pool.fill_(0x5A)
    for key, nb in sizes.items():
        nb = int(-(-nb // 256) * 256)
        per = {}
        for blocks, unroll in READ_CONFIGS:
            n_copies = max(2, min(64, (1 << 30) // nb))
            calls = [w4.bind_ceiling_read(pool[i * nb:(i + 1) * nb], nb, blocks, unroll) for i in range(n_copies)]
            t = _time_calls(torch, calls, max(2 * n_copies, 20))
            per[f"b{blocks}_u{unroll}"] = {"us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1)}
        best = max(per.values(), key=lambda r: r["GBps"])
        res["read_stream"][key] = {"bytes": nb, "best_GBps": best["GBps"], "best_us": best["us"],
                                   "frac_of_8TBps": round(best["GBps"] / HBM_PEAK_GBS, 4), "configs": per}
        log(f"read stream {key}: {best['GBps']} GB/s ({best['us']} us)")
    del pool
    gen = torch.Generator(device="cpu").manual_seed(0)
    n_ops = 1 << 20  # 16 MB of operand chunks
    ops = {
        ("f16", "const"): torch.full((n_ops // 2,), 1.0, dtype=torch.float16),
        ("f16", "random"): torch.randn((n_ops // 2,), generator=gen).to(torch.float16),
        ("i8", "const"): torch.full((n_ops,), 1, dtype=torch.int8),
        ("i8", "random"): torch.randint(-127, 128, (n_ops,), generator=gen, dtype=torch.int8),
    }
    for (kind, data), t_host in ops.items():
        buf = t_host.view(torch.uint8).to(dev)
        per = {}
        # the same work per call at every grid (about 2.5 ms at the random-operand rate),
        # so that the grids compare at the same clock state
        for blocks in (256, 512, 1024, 2048):
            call, flops = w4.bind_ceiling_mfma(buf, 0 if kind == "f16" else 1, 32000 * 256 // blocks, blocks)
            t = _time_calls(torch, [call], 6)
            per[f"b{blocks}"] = round(flops / t / 1e12, 1)
        # a short burst (0.3 ms) before the clock settles, for context
        call, flops = w4.bind_ceiling_mfma(buf, 0 if kind == "f16" else 1, 4000, 256)
        burst = round(flops / _time_calls(torch, [call], 6) / 1e12, 1)
        best = max(per.values())
        peak = F16_PEAK_TFLOPS if kind == "f16" else I8_PEAK_TOPS
        res["mfma"][f"{kind}_{data}"] = {"best_T": best, "frac_of_spec": round(best / peak, 4), "by_blocks": per,
                                         "short_burst_T": burst, "unit": "TFLOP/s" if kind == "f16" else "TOP/s"}
        log(f"mfma {kind} {data}: {best} T/s")
    return res


def _copy_bandwidth(torch, dev, nbytes=1 << 30, iters=5):
    """Read + write bytes per second of torch's device copy of nbytes (context for the
    HBM fraction: the bandwidth a plain streaming kernel reaches here)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / iters
    del a, b
    return 2 * nbytes / t / 1e9


def _time_calls(torch, calls, iters, warm_s=0.03):
    """Average time per call of a list of bound calls run round robin (HIP events), after
    running them for about warm_s seconds so that the clocks are in their steady state
    (the compute-bound GEMMs read ~7 % slower right after an idle gap)."""
    for fn in calls[: min(len(calls), 4)]:
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_s
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            calls[i % len(calls)]()
            i += 1
        torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    n = 0
    for it in range(iters):
        calls[it % len(calls)]()
        n += 1
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / n


def detail(args, dev, torch, np, synth, w4, host, packed):
    out = {}
    it = args.detail_iters
    # single M=8 GEMM (K=N=4096), rotated over 16 copies (8.9 MB each)
    log("detail: single M=8 GEMM")
    inp = synth.make_linear(8, 4096, 4096, seed=0, outliers=False)
    qw, sc, qz = w4.awq_pack(inp.w.to(dev))
    x = inp.x.to(dev)
    y = torch.empty((8, 4096), dtype=torch.float16, device=dev)
    calls = [w4.bind_awq_gemm(x, *rotated_awq(qw, sc, qz, r), y) for r in range(64)]
    t = _time_calls(torch, calls, max(it, 64) * 4)
    b = awq_bytes(8, 4096, 4096)
    out["single_m8_4096"] = {"us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1),
                             "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 3)}
    del calls, qw, sc, qz
    # batch crossover sweep K=5120, N=13824
    log("detail: crossover sweep")
    inp = synth.make_linear(256, 13824, 5120, seed=0, outliers=True)
    qw, sc, qz = w4.awq_pack(inp.w.to(dev))
    copies = [rotated_awq(qw, sc, qz, r) for r in range(16)]
    sweep = {}
    for M in (1, 2, 8, 16, 32, 64, 128, 256):
        x = inp.x[:M].contiguous().to(dev)
        y = torch.empty((M, 13824), dtype=torch.float16, device=dev)
        calls = [w4.bind_awq_gemm(x, *c, y) for c in copies]
        t = _time_calls(torch, calls, max(it, 32))
        b = awq_bytes(M, 13824, 5120)
        fl = 2.0 * M * 13824 * 5120
        sweep[f"M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1), "TFLOPs": round(fl / t / 1e12, 2),
                          "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 3),
                          "frac_f16": round(fl / t / 1e12 / F16_PEAK_TFLOPS, 4)}
    out["crossover_5120x13824"] = sweep
    del copies, qw, sc, qz
    # prefill M=4096
    log("detail: prefill")
    pre = {}
    for (K, N) in ((5120, 27648), (5120, 5120), (13824, 5120)):
        name = {(5120, 27648): "gate_up", (5120, 5120): "o", (13824, 5120): "down"}[(K, N)]
        x = synth.make_activations(4096, K, seed=4096, rms_spread=True).to(dev)
        y = torch.empty((4096, N), dtype=torch.float16, device=dev)
        calls = [w4.bind_awq_gemm(x, *packed[name][r], y) for r in range(len(packed[name]))]
        t = _time_calls(torch, calls, max(4, it // 2))
        fl = 2.0 * 4096 * N * K
        pre[f"{K}x{N}"] = {"us": round(t * 1e6, 1), "TFLOPs": round(fl / t / 1e12, 1),
                           "frac_f16": round(fl / t / 1e12 / F16_PEAK_TFLOPS, 4)}
        del x, y, calls
    out["prefill_13b_M4096"] = pre
    # W4A8
    log("detail: w4a8")
    inp = synth.make_linear(4096, 13824, 5120, seed=0, outliers=True, rms_spread=True, with_gamma=True)
    w8 = {}
    wdev = inp.w.to(dev)
    for group in (-1, 128):
        qw, gs, cs = w4.w4a8_pack(wdev, group)
        copies = [rotated_w4a8(qw, gs, cs, r) for r in range(16)]
        for M in (1, 16, 256, 4096):
            x = inp.x[:M].contiguous().to(dev)
            xq = torch.empty((M, 5120), dtype=torch.int8, device=dev)
            sa = torch.empty((M,), dtype=torch.float32, device=dev)
            qa = w4.bind_w4a8_quant_act(x, inp.gamma.to(dev), xq, sa)
            qa()
            # the quantizer timed over 8 rotated copies of X (336 MB at M = 4096: beyond
            # the 256 MB last-level cache, so the M = 4096 figure is HBM-bound)
            xs_rot = [torch.roll(x, r, 0).contiguous() for r in range(8)]
            qas = [w4.bind_w4a8_quant_act(xr, inp.gamma.to(dev), xq, sa) for xr in xs_rot]
            y = torch.empty((M, 13824), dtype=torch.float16, device=dev)
            calls = [w4.bind_w4a8_gemm(xq, sa, c[0], c[1], c[2], y, group) for c in copies]
            t = _time_calls(torch, calls, max(it, 16) if M < 4096 else max(4, it // 2))
            tq = _time_calls(torch, qas, 16)
            del xs_rot, qas
            b = w4a8_bytes(M, 13824, 5120, group > 0)
            ops = 2.0 * M * 13824 * 5120
            w8[f"{'g128' if group > 0 else 'pc'}_M{M}"] = {
                "gemm_us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1), "TOPs": round(ops / t / 1e12, 2),
                "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 3), "frac_i8": round(ops / t / 1e12 / I8_PEAK_TOPS, 4),
                "frac_f16": round(ops / t / 1e12 / F16_PEAK_TFLOPS, 4), "quant_act_us": round(tq * 1e6, 2)}
        del copies, qw, gs, cs
    out["w4a8_5120x13824"] = w8
    # W8A8 on the same shape (row-major int8 weights, per-channel scales)
    log("detail: w8a8")
    w88 = {}
    qw8, cs8 = w4.w8a8_pack(wdev)
    copies8 = [(torch.roll(qw8, 7 * r, 0).contiguous(), torch.roll(cs8, 112 * r, 0).contiguous()) for r in range(8)]
    for M in (1, 16, 256, 4096):
        x = inp.x[:M].contiguous().to(dev)
        xq, sa = w4.w4a8_quant_act(x, inp.gamma.to(dev))
        y = torch.empty((M, 13824), dtype=torch.float16, device=dev)
        calls = [w4.bind_w8a8_gemm(xq, sa, c[0], c[1], y) for c in copies8]
        t = _time_calls(torch, calls, max(it, 16) if M < 4096 else max(4, it // 2))
        b = 13824 * 5120 + 2 * 13824 + M * 5120 + 4 * M + 2 * M * 13824
        ops = 2.0 * M * 13824 * 5120
        w88[f"M{M}"] = {"gemm_us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1), "TOPs": round(ops / t / 1e12, 2),
                        "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 3), "frac_i8": round(ops / t / 1e12 / I8_PEAK_TOPS, 4)}
    del copies8, qw8, cs8
    out["w8a8_5120x13824"] = w88
    # SiLU-gated quantization of the down projection's input (I = 13824), 4 rotated inputs
    log("detail: silu_mul_quant")
    smq = {}
    I = 13824
    for M in (1, 16, 256, 4096):
        nbuf = 4 if M < 4096 else 2  # 2 x 226 MB at M = 4096: beyond the last-level cache
        gus = [synth.make_activations(M, 2 * I, seed=M + r, rms_spread=True).to(dev) for r in range(nbuf)]
        xq = torch.empty((M, I), dtype=torch.int8, device=dev)
        sa = torch.empty((M,), dtype=torch.float32, device=dev)
        calls = [w4.bind_w4a8_silu_mul_quant(g, xq, sa) for g in gus]
        t = _time_calls(torch, calls, max(it, 16))
        b = M * (2 * I * 2 + I + 4)
        smq[f"M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1),
                        "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 3)}
        del gus
    out["silu_mul_quant_I13824"] = smq
    # W4A16 variants: per-channel and symmetric weights on the same kernels
    log("detail: w4a16 variants")
    var = {}
    for (K, N) in ((5120, 27648), (5120, 5120)):
        w = synth.make_linear(0, N, K, seed=0, outliers=True).w.to(dev)
        for group, sym in ((128, False), (-1, False), (128, True), (-1, True), (64, False), (32, False)):
            pack = w4.awq_pack_sym if sym else w4.awq_pack
            qw, sc, qz = pack(w, group)
            copies = [rotated_awq(qw, sc, qz, r) for r in range(4)]
            for M in ((1, 16) if N > 8192 else (4096,)):
                x = synth.make_activations(M, K, seed=M, rms_spread=True).to(dev)
                y = torch.empty((M, N), dtype=torch.float16, device=dev)
                calls = [w4.bind_awq_gemm(x, *c, y, group) for c in copies]
                t = _time_calls(torch, calls, max(it, 16) if M < 4096 else max(4, it // 2))
                ngr = 1 if group < 0 else K // group
                b = N * K / 2 + 2.5 * N * ngr + 2 * M * K + 2 * M * N
                key = f"{'pc' if group < 0 else f'g{group}'}_{'sym' if sym else 'asym'}_{K}x{N}_M{M}"
                var[key] = {"us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1),
                            "TFLOPs": round(2.0 * M * N * K / t / 1e12, 1)}
            del copies, qw, sc, qz
        del w
    out["w4a16_variants"] = var
    return out


def cpu_baseline(np, synth, host, min_seconds=10.0, max_steps=8):
    """The oracle (numpy dequant + fp64 matmul) on whole decode steps -- the 4 projections
    at M = 1, 4 and 16 (12 GEMMs), packed weights prepared untimed -- repeated until about
    min_seconds of CPU work (at most max_steps steps)."""
    import oracle.ref as ora
    from threadpoolctl import threadpool_info

    log("cpu baseline (oracle)")
    packed = {}
    for name, (K, N) in synth.LLAMA2_13B.items():
        c, s, z = ora.quantize_asym(host[name].w.numpy(), G)
        packed[name] = ora.pack_awq(c, s, z)
    tot_b = 0.0
    tot_t = 0.0
    steps = 0
    while steps < max_steps and (steps == 0 or tot_t < min_seconds):
        for name, (K, N) in synth.LLAMA2_13B.items():
            qw, sg, qz = packed[name]
            for M in (1, 4, 16):
                x = host[name].x[:M].numpy()
                t0 = time.perf_counter()
                wd = ora.dequant_awq(qw, sg, qz, K, G)
                ora.linear_ref(x, wd)
                tot_t += time.perf_counter() - t0
                tot_b += awq_bytes(M, N, K)
                del wd
        steps += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(tot_b / tot_t / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} decode steps: QKV/O/gate+up/down at M=1,4,16 (12 GEMMs each), numpy fp64 dequant "
                      f"+ BLAS matmul, {tot_t:.1f} s", "host_cpu_count": os.cpu_count()}


if __name__ == "__main__":
    main()
