#!/usr/bin/env python3
"""Benchmark of the GPTQ weight-only GEMM on one MI355X.

Metric: "GPTQ W4A16 GEMM: weight GB/s at M=1 and TFLOP/s at M=2048, % of
roofline".  A step is one decode pass over the four Llama-7B-shaped layers
(qkv 4096->12288, o_proj 4096->4096, gate_up 4096->22016, down 11008->4096) at
M=1, 4-bit g128 symmetric GPTQv1, synthetic seeded weights quantized on the
GPU by the library's own quantizer.  `value` = packed weight bytes (qweight +
qzeros + scales) per step / step time.  Distinct weight copies (>= 1 GB in
total) are rotated so the 256 MB Infinity Cache cannot serve them.

The JSON line also carries:
  roofline      the decode kernel: algorithmic bytes per launch (weights + x +
                y) / its mean launch time (HIP events around replays of a HIP
                graph of that layer's launches over the rotated copies),
                against 8 TB/s;
  prefill       the 70B-MLP M=2048 GEMMs (4-bit g128 sym v1, 8-bit g128 asym
                v2): TFLOP/s against 2.5 PFLOP/s dense fp16 MFMA;
  cpu_baseline  the CPU oracle (numpy, fp64) on a bounded column slice of the
                qkv layer, same unit.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
ROTATE_BYTES = 1 << 30          # rotate >= 1 GiB of distinct weight copies


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-cols", type=int, default=2048,
                   help="columns of the qkv layer the CPU oracle processes")
    return p.parse_args()


def layer_bytes(K, N, bits, gs):
    G = K // gs
    return K * bits // 8 * N + G * N * bits // 8 + G * N * 2   # qweight + qzeros + scales


def make_layer(torch, gq, wl, layer, M, dev):
    from workload import draw_workload_layer
    d = draw_workload_layer(wl, layer, M, seed=0)
    w = torch.from_numpy(d.W).to(dev)
    gi = None if d.g_idx is None else torch.from_numpy(d.g_idx).to(dev)
    qw, qz, sc = gq.quantize(w, gi, wl.bits, wl.group_size, wl.sym, wl.is_v2)
    del w
    x = torch.from_numpy(d.x).to(dev)
    return dict(qweight=qw, qzeros=qz, scales=sc, g_idx=gi, x=x, K=layer.K, N=layer.N)


def bench_decode(torch, gq, args, dev):
    """Decode step timing.  Launches are captured in HIP graphs so the Python
    binding's per-call overhead stays out of the timed region: one graph holds
    R steps (R rotated weight copies x 4 layers); per-layer graphs hold R launches
    of one layer and give the kernel's mean launch time."""
    from workload import WORKLOADS
    wl = WORKLOADS["llama7b_decode_w4g128"]
    base = [make_layer(torch, gq, wl, l, 1, dev) for l in wl.layers]
    wbytes = sum(layer_bytes(L["K"], L["N"], wl.bits, wl.group_size) for L in base)
    copies = max(1, -(-ROTATE_BYTES // wbytes))
    sets = [base] + [[{**L, "qweight": L["qweight"].clone(), "qzeros": L["qzeros"].clone(),
                       "scales": L["scales"].clone()} for L in base] for _ in range(copies - 1)]
    outs = [torch.empty((1, L["N"]), dtype=torch.float16, device=dev) for L in base]

    def launch(r, j):
        L = sets[r][j]
        gq.gemm(L["x"], L["qweight"], L["qzeros"], L["scales"], None, wl.bits, wl.group_size, wl.is_v2,
                out=outs[j])

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(max(args.warmup, 1)):          # also allocates the split-K workspace of `side`
            for j in range(len(base)):
                launch(i % copies, j)
    torch.cuda.synchronize()

    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all, stream=side):
        for r in range(copies):
            for j in range(len(base)):
                launch(r, j)
    g_layer = []
    for j in range(len(base)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for r in range(copies):
                launch(r, j)
        g_layer.append(g)

    def timed(graph, reps):
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream(dev)
        e0.record(st)
        for _ in range(reps):
            graph.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    replays = max(1, -(-args.steps // copies))
    steps = replays * copies
    ms_per_step = timed(g_all, replays) / steps
    per_layer_ms = [timed(g, replays) / steps for g in g_layer]

    alg = [layer_bytes(L["K"], L["N"], wl.bits, wl.group_size) + 2 * L["K"] + 2 * L["N"] for L in base]
    mean_launch_ms = float(np.mean(per_layer_ms))
    achieved = (sum(alg) / len(alg)) / (mean_launch_ms * 1e-3) / 1e9
    layers = [{"layer": l.name, "K": l.K, "N": l.N, "alg_bytes": a, "us": round(t * 1e3, 2),
               "GBps": round(a / (t * 1e-3) / 1e9, 1)} for l, a, t in zip(wl.layers, alg, per_layer_ms)]
    del g_all, g_layer
    return dict(wl=wl, wbytes=wbytes, copies=copies, ms_per_step=ms_per_step, achieved=achieved, steps=steps,
                mean_launch_us=mean_launch_ms * 1e3, layers=layers, base=base)


def bench_prefill(torch, gq, args, dev):
    from workload import WORKLOADS
    res = []
    for name in ("mlp70b_prefill_w4g128", "mlp70b_prefill_w8g128"):
        wl = WORKLOADS[name]
        for layer in wl.layers:
            L = make_layer(torch, gq, wl, layer, 2048, dev)
            out = torch.empty((2048, layer.N), dtype=torch.float16, device=dev)
            run = lambda: gq.gemm(L["x"], L["qweight"], L["qzeros"], L["scales"], None, wl.bits,
                                  wl.group_size, wl.is_v2, out=out)
            for _ in range(2):
                run()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.prefill_steps):
                run()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.prefill_steps
            flops = 2.0 * 2048 * layer.K * layer.N
            tf = flops / (ms * 1e-3) / 1e12
            res.append({"workload": name, "layer": layer.name, "M": 2048, "K": layer.K, "N": layer.N,
                        "bits": wl.bits, "ms": round(ms, 4), "TFLOPs": round(tf, 1),
                        "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)})
            del L, out
            torch.cuda.empty_cache()
    return res


def copy_ceiling(torch, dev):
    """Plain device copy of 1 GiB: read + write GB/s (context for the HBM roofline)."""
    a = torch.empty(1 << 29, dtype=torch.float16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    return 2 * a.numel() * 2 / (ms * 1e-3) / 1e9


def cpu_baseline(args):
    """The oracle (dequant from packed arrays + fp64 matmul) on a column slice of
    the qkv layer; inputs quantized by the oracle itself from the same draw."""
    import oracle
    from workload import WORKLOADS, draw_workload_layer
    wl = WORKLOADS["llama7b_decode_w4g128"]
    layer = wl.layers[0]
    d = draw_workload_layer(wl, layer, 1, seed=0)
    ncols = min(args.cpu_sample_cols, layer.N)
    W = np.ascontiguousarray(d.W[:, :ncols])
    L = oracle.quantize_layer(W, wl.bits, wl.group_size, wl.sym, wl.is_v2)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, wl.bits, wl.group_size, wl.is_v2,
                             layer.K, ncols)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or reps >= 20:
            break
    sec = el / reps
    gbps = layer_bytes(layer.K, ncols, wl.bits, wl.group_size) / sec / 1e9
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:
        pass
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"qkv layer K={layer.K}, first {ncols} of {layer.N} columns, M=1; "
                      f"{reps} run(s), {sec:.2f} s each (numpy fp64 dequant + matmul; elementwise ops "
                      f"single-threaded, BLAS up to {threads} threads)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import weight_only_bit_gptq_amd as gq
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    gq.library()

    dec = bench_decode(torch, gq, args, dev)
    print(f"# decode: {dec['ms_per_step'] * 1e3:.2f} us/step, layers: {dec['layers']}", file=sys.stderr, flush=True)
    del dec["base"]
    torch.cuda.empty_cache()
    ceiling = copy_ceiling(torch, dev)
    prefill = None if args.no_prefill else bench_prefill(torch, gq, args, dev)
    if prefill:
        print(f"# prefill: {prefill}", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args)

    wl = dec["wl"]
    value = dec["wbytes"] / (dec["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": "GPTQ W4A16 GEMM: weight GB/s at M=1 and TFLOP/s at M=2048, % of roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": dec["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) weights, min/max quantized on the GPU; N(0,1) fp16 x)",
        "config": {"workload": wl.name, "layers": [f"{l.name} {l.K}->{l.N}" for l in wl.layers], "M": 1,
                   "bits": wl.bits, "group_size": wl.group_size, "sym": wl.sym, "format": "v2" if wl.is_v2 else "v1",
                   "weight_bytes_per_step": dec["wbytes"], "rotated_copies": dec["copies"]},
        "roofline": {"bound": "hbm", "achieved": round(dec["achieved"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec["achieved"] / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "decode_kernel<4,false,1,8>", "mean_launch_us": round(dec["mean_launch_us"], 3),
                     "per_layer": dec["layers"]},
        "copy_GBps": round(ceiling, 1),
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
