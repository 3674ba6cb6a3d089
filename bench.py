#!/usr/bin/env python3
"""Benchmark of the GPTQ weight-only GEMM on one MI355X.

Metric: "GPTQ W4A16 GEMM: weight GB/s at M=1 and TFLOP/s at M=2048, % of
roofline".  A step is one decode pass over the four Llama-7B-shaped layers
(qkv 4096->12288, o_proj 4096->4096, gate_up 4096->22016, down 11008->4096) at
M=1, 4-bit g128 symmetric GPTQv1, synthetic seeded weights quantized on the
GPU by the library's own quantizer, qweight then re-laid out once into the
tiled layout (gptq_repack_tiled, untimed).  `value` = packed weight bytes
(qweight + qzeros + scales) per step / step time.  Distinct weight copies
(>= 1 GB in total) are rotated so the 256 MB Infinity Cache cannot serve them.
The same step on the checkpoint qweight layout is reported beside it.

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

Counter passes (HBM traffic of the decode kernel, see `--pmc-driver`):
  rocprofv3 --pmc FETCH_SIZE -d D/fetch -o run -f csv -- python3 bench.py --pmc-driver
  rocprofv3 --pmc WRITE_SIZE -d D/write -o run -f csv -- python3 bench.py --pmc-driver
  python3 bench.py --summarize-pmc D/fetch/run_counter_collection.csv D/write/run_counter_collection.csv
The summary goes to profiles/; `roofline.traffic` is read from it while the
decode sources still hash to the value recorded there (null otherwise).

Counter pass (MFMA utilisation of the prefill kernel, see `--pmc-prefill-driver`):
  rocprofv3 --pmc MfmaUtil GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA --kernel-trace -d D/mfma -o run -f csv \
      -- python3 bench.py --pmc-prefill-driver
  python3 bench.py --summarize-prefill-pmc D/mfma/run_counter_collection.csv D/mfma/run_kernel_trace.csv
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama7b_w4g128_hbm_traffic.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_mlp70b_mfma_util.txt")
# sources that decide the decode kernel's code and launch shapes
DECODE_SOURCES = ["weight_only_bit_gptq_amd/csrc/decode.hip", "weight_only_bit_gptq_amd/csrc/gptq_device.hpp",
                  "weight_only_bit_gptq_amd/csrc/gptq_kernels.hpp", "weight_only_bit_gptq_amd/csrc/gptq_api.cpp"]
PMC_COPY_BYTES = 256 << 20      # plain copy of known size that calibrates FETCH_SIZE / WRITE_SIZE

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 (and bf16) MFMA
ROTATE_BYTES = 1 << 30          # rotate >= 1 GiB of distinct weight copies


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--warm-seconds", type=float, default=0.5,
                   help="untimed GPU work before each timed region (MI355X raises its clocks over "
                        "hundreds of milliseconds of load; measured without it, prefill reads ~15%% low)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-checkpoint-layout", action="store_true",
                   help="skip the decode step on the checkpoint qweight layout (reported beside the tiled one)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16", action="store_true",
                   help="skip the bfloat16-activation lines (decode layers and 4-bit prefill)")
    p.add_argument("--cpu-sample-cols", type=int, default=12288,
                   help="columns of the qkv layer the CPU oracle processes (default: all)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="repeat the oracle on the sample until this much CPU time has passed")
    p.add_argument("--pmc-driver", action="store_true",
                   help="only launch each decode layer 3 times and a plain copy, for a rocprofv3 --pmc pass")
    p.add_argument("--pmc-prefill-driver", action="store_true",
                   help="only launch each 70B-MLP prefill layer twice, for a rocprofv3 --pmc pass")
    p.add_argument("--summarize-prefill-pmc", nargs=2, metavar=("COUNTER_CSV", "TRACE_CSV"),
                   help="write the prefill MFMA-utilisation summary to profiles/ from a --pmc-prefill-driver pass")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the HBM traffic summary from two counter passes (no GPU needed)")
    return p.parse_args()


def decode_sources_hash():
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Per-layer HBM bytes per launch from the committed counter summary, or
    None when it is missing or was taken on other decode sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [l for l in f if l.startswith("json: ")]
        rec = json.loads(lines[-1][len("json: "):])
    except (OSError, IndexError, ValueError):
        return None
    return rec if rec.get("sources_sha256") == decode_sources_hash() else None


def layer_bytes(K, N, bits, gs):
    G = K // gs
    return K * bits // 8 * N + G * N * bits // 8 + G * N * 2   # qweight + qzeros + scales


def make_layer(torch, gq, wl, layer, M, dev, tiled=False):
    from workload import draw_workload_layer
    d = draw_workload_layer(wl, layer, M, seed=0)
    w = torch.from_numpy(d.W).to(dev)
    gi = None if d.g_idx is None else torch.from_numpy(d.g_idx).to(dev)
    qw, qz, sc = gq.quantize(w, gi, wl.bits, wl.group_size, wl.sym, wl.is_v2)
    del w
    if tiled:                      # one-time re-layout at load (not timed)
        qw = gq.repack_tiled(qw, wl.bits)
    x = torch.from_numpy(d.x).to(dev)
    return dict(qweight=qw, qzeros=qz, scales=sc, g_idx=gi, x=x, K=layer.K, N=layer.N)


def to_bf16(torch, L):
    """The same layer with bfloat16 activations: x and scales rounded to bfloat16."""
    return {**L, "x": L["x"].to(torch.bfloat16), "scales": L["scales"].to(torch.bfloat16)}


def bench_decode(torch, gq, args, dev, tiled, bf16=False):
    """Decode step timing.  Launches are captured in HIP graphs so the Python
    binding's per-call overhead stays out of the timed region: one graph holds
    R steps (R rotated weight copies x 4 layers); per-layer graphs hold R launches
    of one layer and give the kernel's mean launch time.  `tiled`: qweight in
    the tiled layout (repacked once at load), else the checkpoint layout.
    `bf16`: bfloat16 activations and scales (gptq_gemm_bf16)."""
    from workload import WORKLOADS
    wl = WORKLOADS["llama7b_decode_w4g128"]
    base = [make_layer(torch, gq, wl, l, 1, dev, tiled) for l in wl.layers]
    if bf16:
        base = [to_bf16(torch, L) for L in base]
    adt = torch.bfloat16 if bf16 else torch.float16
    wbytes = sum(layer_bytes(L["K"], L["N"], wl.bits, wl.group_size) for L in base)
    copies = max(1, -(-ROTATE_BYTES // wbytes))
    sets = [base] + [[{**L, "qweight": L["qweight"].clone(), "qzeros": L["qzeros"].clone(),
                       "scales": L["scales"].clone()} for L in base] for _ in range(copies - 1)]
    outs = [torch.empty((1, L["N"]), dtype=adt, device=dev) for L in base]

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

    def warm(graph):
        # untimed replays until the clocks have settled (see --warm-seconds)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.warm_seconds:
            for _ in range(20):
                graph.replay()
            torch.cuda.synchronize()

    replays = max(1, -(-args.steps // copies))
    steps = replays * copies
    warm(g_all)
    ms_per_step = timed(g_all, replays) / steps
    per_layer_ms = [timed(g, replays) / steps for g in g_layer]

    alg = [layer_bytes(L["K"], L["N"], wl.bits, wl.group_size) + 2 * L["K"] + 2 * L["N"] for L in base]
    mean_launch_ms = float(np.mean(per_layer_ms))
    achieved = (sum(alg) / len(alg)) / (mean_launch_ms * 1e-3) / 1e9
    kernels = [gq.describe(L["x"], L["qweight"], L["qzeros"], L["scales"], None, wl.bits, wl.group_size, wl.is_v2,
                           out=o) for L, o in zip(base, outs)]
    layers = [{"layer": l.name, "K": l.K, "N": l.N, "kernel": kn, "alg_bytes": a, "us": round(t * 1e3, 2),
               "GBps": round(a / (t * 1e-3) / 1e9, 1)}
              for l, kn, a, t in zip(wl.layers, kernels, alg, per_layer_ms)]
    del g_all, g_layer
    return dict(wl=wl, wbytes=wbytes, copies=copies, ms_per_step=ms_per_step, achieved=achieved, steps=steps,
                mean_launch_us=mean_launch_ms * 1e3, layers=layers, base=base)


def bench_prefill(torch, gq, args, dev, bf16=False):
    """Prefill GEMM timing per layer (plus, for the 4-bit workload, the vendor
    dense GEMM in the same activation type on the same shape, as context).
    fp16: qweight in the tiled layout, the same re-laid-out copy the decode
    step reads (4-bit tiled words hold their fields in pair order, which the
    prefill kernel unpacks with fewer instructions).  `bf16`: bfloat16
    activations and scales, 4-bit workload only, checkpoint layout (the only
    one bfloat16 reads)."""
    from workload import WORKLOADS
    res = []
    adt = torch.bfloat16 if bf16 else torch.float16
    names = ("mlp70b_prefill_w4g128",) if bf16 else ("mlp70b_prefill_w4g128", "mlp70b_prefill_w8g128")
    for name in names:
        wl = WORKLOADS[name]
        for layer in wl.layers:
            L = make_layer(torch, gq, wl, layer, 2048, dev, tiled=not bf16)
            if bf16:
                L = to_bf16(torch, L)
            out = torch.empty((2048, layer.N), dtype=adt, device=dev)
            run = lambda: gq.gemm(L["x"], L["qweight"], L["qzeros"], L["scales"], None, wl.bits,
                                  wl.group_size, wl.is_v2, out=out)
            t0 = time.perf_counter()
            while True:                       # untimed warm-up (see --warm-seconds)
                for _ in range(5):
                    run()
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= args.warm_seconds:
                    break
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
            row = {"workload": name, "layer": layer.name, "M": 2048, "K": layer.K, "N": layer.N,
                   "bits": wl.bits, "qweight_layout": "checkpoint" if bf16 else "tiled", "ms": round(ms, 4),
                   "TFLOPs": round(tf, 1), "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
            if name == "mlp70b_prefill_w4g128":
                # context: the vendor dense GEMM (torch.matmul) on the same shape, unquantized W
                W = torch.randn((layer.K, layer.N), dtype=adt, device=dev)
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < args.warm_seconds:
                    for _ in range(5):
                        torch.matmul(L["x"], W, out=out)
                    torch.cuda.synchronize()
                a.record()
                for _ in range(args.prefill_steps):
                    torch.matmul(L["x"], W, out=out)
                b.record()
                torch.cuda.synchronize()
                key = "dense_bf16_matmul_TFLOPs" if bf16 else "dense_fp16_matmul_TFLOPs"
                row[key] = round(flops / (a.elapsed_time(b) / args.prefill_steps * 1e-3) / 1e12, 1)
                del W
            res.append(row)
            del L, out
            torch.cuda.empty_cache()
    return res


def bench_decode_configs(torch, gq, args, dev):
    """The other decode workloads (2-bit g64 asym v2 with outliers at M = 1, 4,
    16; 3-bit g128 act-order at M = 16, rows sorted by group once at load and
    x gathered per call), tiled layout: per-layer launch time
    from a graph of launches over rotated weight copies, and algorithmic
    bytes (weights + g_idx + x + y) per launch against 8 TB/s."""
    from workload import WORKLOADS
    res = []
    for name in ("lowbit_decode_w2g64", "actorder_decode_w3g128"):
        wl = WORKLOADS[name]
        for layer in wl.layers:
            L = make_layer(torch, gq, wl, layer, max(wl.Ms), dev, tiled=not wl.act_order)
            perm = None
            if wl.act_order:               # rows sorted by group once at load, x gathered per call
                qs, perm = gq.sort_act_order(L["qweight"], L["g_idx"], wl.bits, wl.group_size)
                L["qweight"] = gq.repack_tiled(qs, wl.bits)
                del qs
            wb = layer_bytes(layer.K, layer.N, wl.bits, wl.group_size) + (4 * layer.K if wl.act_order else 0)
            copies = max(2, -(-ROTATE_BYTES // wb))
            sets = [L["qweight"]] + [L["qweight"].clone() for _ in range(copies - 1)]
            for M in wl.Ms:
                x = L["x"][:M].contiguous()
                out = torch.empty((M, layer.N), dtype=torch.float16, device=dev)
                if perm is None:
                    run = lambda qw: gq.gemm(x, qw, L["qzeros"], L["scales"], None, wl.bits, wl.group_size,
                                             wl.is_v2, out=out)
                else:
                    run = lambda qw: gq.gemm_sorted(x, qw, L["qzeros"], L["scales"], perm, wl.bits, wl.group_size,
                                                    wl.is_v2, out=out)
                side = torch.cuda.Stream(dev)
                side.wait_stream(torch.cuda.current_stream(dev))
                with torch.cuda.stream(side):
                    for qw in sets:
                        run(qw)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    for qw in sets:
                        run(qw)
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < args.warm_seconds / 4:
                    for _ in range(10):
                        g.replay()
                    torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                reps = 20
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
                alg = wb + 2 * M * layer.K + 2 * M * layer.N
                res.append({"workload": name, "layer": f"{layer.name} {layer.K}->{layer.N}", "M": M,
                            "kernel": ("x gathered by perm, then " if perm is not None else "") +
                                      gq.describe(x, sets[0], L["qzeros"], L["scales"], None, wl.bits,
                                                  wl.group_size, wl.is_v2, out=out),
                            "us": round(us, 2), "GBps": round(alg / (us * 1e-6) / 1e9, 1),
                            "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
                del g
            del L, sets
            torch.cuda.empty_cache()
    return res


def bench_moe(torch, gq, args, dev):
    """Grouped decode (gptq_moe_gemm) on a Mixtral-class expert layer: 8 experts
    4096 -> 14336, 4-bit g128 sym v1, 16 tokens routed top-2 (seeded), weight
    copies rotated past the Infinity Cache.  Reports weight GB/s over the
    experts that received tokens (all of them read once per launch)."""
    E, K, N, bits, gs = 8, 4096, 14336, 4, 128
    rng = np.random.default_rng(0)
    picks = np.array([rng.choice(E, size=2, replace=False) for _ in range(16)]).ravel()
    counts = np.bincount(picks, minlength=E)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=dev)
    T = int(counts.sum())
    gen = torch.Generator(device=dev).manual_seed(0)
    qws, qzs, scs = [], [], []
    for _ in range(E):
        w = torch.randn((K, N), generator=gen, device=dev, dtype=torch.float32) * 0.02
        qw, qz, sc = gq.quantize(w, None, bits, gs, True, False)
        qws.append(qw), qzs.append(qz), scs.append(sc)
        del w
    base = (torch.stack(qws), torch.stack(qzs), torch.stack(scs))
    del qws, qzs, scs
    x = torch.randn((T, K), generator=gen, device=dev, dtype=torch.float32).half()
    out = torch.empty((T, N), dtype=torch.float16, device=dev)
    active = int((counts > 0).sum())
    wbytes = active * layer_bytes(K, N, bits, gs)
    copies = max(2, -(-ROTATE_BYTES // (E * layer_bytes(K, N, bits, gs))))
    sets = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
    mt = int(counts.max())
    run = lambda st: gq.moe_gemm(x, st[0], st[1], st[2], None, offsets, mt, bits, gs, False, out=out)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for st in sets:
            run(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for st in sets:
            run(st)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.warm_seconds:     # untimed warm-up
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    del g, sets, base
    torch.cuda.empty_cache()
    return {"workload": "mixtral_expert_w1_w4g128", "experts": E, "K": K, "N": N, "tokens": 16, "top_k": 2,
            "active_experts": active, "us": round(us, 2), "weight_GBps": round(wbytes / (us * 1e-6) / 1e9, 1),
            "frac": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


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
        if el >= args.cpu_seconds or reps >= 200:
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


def pmc_driver(torch, gq, dev):
    """Each decode layer 3 times (distinct weight copies, so no launch finds its
    weights in L2), then a plain copy of PMC_COPY_BYTES; no timing."""
    from workload import WORKLOADS
    wl = WORKLOADS["llama7b_decode_w4g128"]
    for layer in wl.layers:
        L = make_layer(torch, gq, wl, layer, 1, dev, tiled=True)
        out = torch.empty((1, layer.N), dtype=torch.float16, device=dev)
        copies = [(L["qweight"].clone(), L["qzeros"].clone(), L["scales"].clone()) for _ in range(3)]
        torch.cuda.synchronize()
        for qw, qz, sc in copies:
            gq.gemm(L["x"], qw, qz, sc, None, wl.bits, wl.group_size, wl.is_v2, out=out)
        torch.cuda.synchronize()
        print(f"{layer.name}: {gq.describe(L['x'], qw, qz, sc, None, wl.bits, wl.group_size, wl.is_v2, out=out)}",
              flush=True)
        del L, copies
    a = torch.ones(PMC_COPY_BYTES // 2, dtype=torch.float16, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("pmc driver done", flush=True)


PREFILL_WORKLOADS = ("mlp70b_prefill_w4g128", "mlp70b_prefill_w8g128")
MI355X_XCDS = 8


def pmc_prefill_driver(torch, gq, dev):
    """Each 70B-MLP prefill layer (M = 2048, tiled layout) twice on its own weights; no timing."""
    from workload import WORKLOADS
    for name in PREFILL_WORKLOADS:
        wl = WORKLOADS[name]
        for layer in wl.layers:
            L = make_layer(torch, gq, wl, layer, 2048, dev, tiled=True)      # as the bench times it
            out = torch.empty((2048, layer.N), dtype=torch.float16, device=dev)
            torch.cuda.synchronize()
            for _ in range(2):
                gq.gemm(L["x"], L["qweight"], L["qzeros"], L["scales"], None, wl.bits, wl.group_size, wl.is_v2,
                        out=out)
            torch.cuda.synchronize()
            print(f"{name} {layer.name}: {gq.describe(L['x'], L['qweight'], L['qzeros'], L['scales'], None, wl.bits, wl.group_size, wl.is_v2, out=out)}",
                  flush=True)
            del L, out
            torch.cuda.empty_cache()
    print("pmc prefill driver done", flush=True)


def summarize_prefill_pmc(counter_csv, trace_csv):
    """MfmaUtil (MFMA busy cycles / (GPU active cycles x SIMDs)), the clock the
    kernel ran at (GRBM_GUI_ACTIVE / kernel duration) and VALU / MFMA
    instruction counts of the second launch of each prefill layer."""
    from workload import WORKLOADS
    vals = {}
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if "prefill_kernel" in r["Kernel_Name"]:
                d = vals.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    dur = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    ids = sorted(vals)
    layers = [(n, l) for n in PREFILL_WORKLOADS for l in WORKLOADS[n].layers]
    if len(ids) != 2 * len(layers):
        raise SystemExit(f"expected {2 * len(layers)} prefill dispatches, got {len(ids)}")
    lines = [
        "# MFMA utilisation of the prefill kernel, 70B-MLP shapes at M=2048 (4-bit g128 sym v1, 8-bit g128 asym",
        "# v2), one MI355X; second of two launches per layer, counters summed over the chip.",
        "# Command (run from /tmp with TMPDIR=/tmp; R = repository root):",
        "#   rocprofv3 --pmc MfmaUtil GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA --kernel-trace -d D/mfma -o run -f csv "
        "-- python3 R/bench.py --pmc-prefill-driver",
        "#   python3 R/bench.py --summarize-prefill-pmc D/mfma/run_counter_collection.csv D/mfma/run_kernel_trace.csv",
        "# MfmaUtil = sum of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) (rocprofv3's derived counter);",
        "# clock = GRBM_GUI_ACTIVE / 8 / kernel duration (the CSV sums the counter over the 8 XCDs);",
        "# TFLOP/s from the kernel duration under the profiler (no warm-up: clocks are still rising).",
        "# SQ_INSTS_VALU counts the MFMA instructions too (so the other VALU per MFMA is the ratio minus 1).",
        "layer | kernel | us | TFLOP/s | clock GHz | MfmaUtil % | SQ_INSTS_VALU / SQ_INSTS_MFMA",
    ]
    rec = []
    for i, (name, layer) in enumerate(layers):
        did = ids[2 * i + 1]
        v = vals[did]
        us = dur[did] / 1e3
        flops = 2.0 * 2048 * layer.K * layer.N
        # GRBM_GUI_ACTIVE has one instance per XCD and the CSV holds their sum: per-XCD cycles are 1/8
        clk = v.get("GRBM_GUI_ACTIVE", 0.0) / MI355X_XCDS / dur[did]
        ratio = v.get("SQ_INSTS_VALU", 0.0) / max(v.get("SQ_INSTS_MFMA", 0.0), 1.0)
        rec.append({"workload": name, "layer": layer.name, "kernel": v["kernel"], "us": round(us, 2),
                    "TFLOPs": round(flops / us / 1e6, 1), "clock_GHz": round(clk, 3),
                    "MfmaUtil": round(v.get("MfmaUtil", float("nan")), 2), "valu_per_mfma": round(ratio, 2)})
        lines.append(f"{name} {layer.name} | {v['kernel']} | {us:.1f} | {flops / us / 1e6:.1f} | {clk:.3f} | "
                     f"{v.get('MfmaUtil', float('nan')):.1f} | {ratio:.2f}")
    lines.append("json: " + json.dumps(rec))
    os.makedirs(os.path.dirname(MFMA_FILE), exist_ok=True)
    with open(MFMA_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(fetch_csv, write_csv):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the decode launches, scaled
    by what the same counters read for the plain copy of PMC_COPY_BYTES."""
    from workload import WORKLOADS
    wl = WORKLOADS["llama7b_decode_w4g128"]

    def rows(path, counter):
        out = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
        out.sort()
        return out

    res = {}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rs = rows(path, counter)
        dec = [r for r in rs if "decode_kernel" in r[1]]
        cop = [r for r in rs if "copyBuffer" in r[1] or "copy" in r[1].lower()]
        if len(dec) != 3 * len(wl.layers) or not cop:
            raise SystemExit(f"{path}: expected {3 * len(wl.layers)} decode dispatches and a copy, "
                             f"got {len(dec)} and {len(cop)}")
        copy_kib = float(np.median([r[3] for r in cop[-3:]]))
        scale = PMC_COPY_BYTES / (copy_kib * 1024.0)
        res[name] = dict(dec=dec, copy_kib=copy_kib, scale=scale)
    layers = []
    for i, layer in enumerate(wl.layers):
        f = res["fetch"]["dec"][3 * i:3 * i + 3]
        w = res["write"]["dec"][3 * i:3 * i + 3]
        fetch = float(np.mean([r[3] for r in f])) * 1024.0 * res["fetch"]["scale"]
        write = float(np.mean([r[3] for r in w])) * 1024.0 * res["write"]["scale"]
        alg = layer_bytes(layer.K, layer.N, wl.bits, wl.group_size) + 2 * layer.K + 2 * layer.N
        layers.append({"layer": layer.name, "kernel": f[0][1], "grid": f[0][2],
                       "fetch_bytes": int(fetch), "write_bytes": int(write), "traffic_bytes": int(fetch + write),
                       "alg_bytes": alg, "traffic_over_alg": round((fetch + write) / alg, 4)})
    rec = {"sources_sha256": decode_sources_hash(), "copy_bytes": PMC_COPY_BYTES,
           "fetch_scale": round(res["fetch"]["scale"], 5), "write_scale": round(res["write"]["scale"], 5),
           "layers": layers}
    lines = [
        "# HBM traffic per launch of the decode kernel, Llama-7B-shaped decode layers",
        "# (M=1, 4-bit, group 128, symmetric, GPTQv1, qweight in the tiled layout), one MI355X.",
        "# Commands (run from /tmp with TMPDIR=/tmp; R = repository root):",
        "#   rocprofv3 --pmc FETCH_SIZE -d D/fetch -o run -f csv -- python3 R/bench.py --pmc-driver",
        "#   rocprofv3 --pmc WRITE_SIZE -d D/write -o run -f csv -- python3 R/bench.py --pmc-driver",
        "#   python3 R/bench.py --summarize-pmc D/fetch/run_counter_collection.csv D/write/run_counter_collection.csv",
        f"# Calibration: a plain copy of {PMC_COPY_BYTES} bytes read FETCH_SIZE {res['fetch']['copy_kib']:.1f} KiB "
        f"and WRITE_SIZE {res['write']['copy_kib']:.1f} KiB;",
        f"# scale factors fetch {rec['fetch_scale']}, write {rec['write_scale']} (bytes per counted byte).",
        "# Per layer: mean over 3 launches on distinct weight copies.",
    ]
    for l in layers:
        lines.append(f"{l['layer']:8s} {l['kernel']}  grid {l['grid']}: fetch {l['fetch_bytes']} B, write "
                     f"{l['write_bytes']} B, traffic {l['traffic_bytes']} B, algorithmic {l['alg_bytes']} B, "
                     f"ratio {l['traffic_over_alg']}")
    lines.append("json: " + json.dumps(rec))
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_prefill_pmc:
        summarize_prefill_pmc(*args.summarize_prefill_pmc)
        return
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
    if args.pmc_driver:
        pmc_driver(torch, gq, dev)
        return
    if args.pmc_prefill_driver:
        pmc_prefill_driver(torch, gq, dev)
        return

    dec = bench_decode(torch, gq, args, dev, tiled=True)
    print(f"# decode (tiled): {dec['ms_per_step'] * 1e3:.2f} us/step, layers: {dec['layers']}", file=sys.stderr,
          flush=True)
    del dec["base"]
    torch.cuda.empty_cache()
    dec_ck = None
    if not args.no_checkpoint_layout:
        dec_ck = bench_decode(torch, gq, args, dev, tiled=False)
        print(f"# decode (checkpoint layout): {dec_ck['ms_per_step'] * 1e3:.2f} us/step, layers: {dec_ck['layers']}",
              file=sys.stderr, flush=True)
        del dec_ck["base"]
    torch.cuda.empty_cache()
    dec_other = bench_decode_configs(torch, gq, args, dev)
    print(f"# other decode configs: {dec_other}", file=sys.stderr, flush=True)
    moe = bench_moe(torch, gq, args, dev)
    print(f"# moe: {moe}", file=sys.stderr, flush=True)
    ceiling = copy_ceiling(torch, dev)
    prefill = None if args.no_prefill else bench_prefill(torch, gq, args, dev)
    if prefill:
        print(f"# prefill: {prefill}", file=sys.stderr, flush=True)
    bf16 = None
    if not args.no_bf16:
        torch.cuda.empty_cache()
        dec_bf = bench_decode(torch, gq, args, dev, tiled=False, bf16=True)
        del dec_bf["base"]
        torch.cuda.empty_cache()
        bf16 = {"decode": {"workload": dec_bf["wl"].name + " with bf16 x and scales (checkpoint layout)",
                           "value": round(dec_bf["wbytes"] / (dec_bf["ms_per_step"] * 1e-3) / 1e9, 1),
                           "ms_per_step": round(dec_bf["ms_per_step"], 5), "achieved": round(dec_bf["achieved"], 1),
                           "frac": round(dec_bf["achieved"] / HBM_PEAK_GBPS, 4),
                           "mean_launch_us": round(dec_bf["mean_launch_us"], 3), "per_layer": dec_bf["layers"]},
                "prefill": None if args.no_prefill else bench_prefill(torch, gq, args, dev, bf16=True)}
        print(f"# bf16: {bf16}", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args)

    wl = dec["wl"]
    value = dec["wbytes"] / (dec["ms_per_step"] * 1e-3) / 1e9
    traffic = read_traffic()
    traffic_bytes = None
    if traffic is not None:
        by_layer = {t["layer"]: t for t in traffic["layers"]}
        if all(l["layer"] in by_layer for l in dec["layers"]):
            for l in dec["layers"]:
                l["traffic_bytes"] = by_layer[l["layer"]]["traffic_bytes"]
            traffic_bytes = int(np.mean([l["traffic_bytes"] for l in dec["layers"]]))
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
                   "weight_bytes_per_step": dec["wbytes"], "rotated_copies": dec["copies"],
                   "qweight_layout": "tiled [N/16][K/32][bits][16], made once at load by gptq_repack_tiled (untimed)"},
        "roofline": {"bound": "hbm", "achieved": round(dec["achieved"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec["achieved"] / HBM_PEAK_GBPS, 4), "traffic": traffic_bytes,
                     "kernel": "gptq::decode_kernel, one instantiation per layer (per_layer[].kernel); achieved = "
                               "mean algorithmic bytes per launch / mean launch time over the 4 layers; traffic = "
                               "mean HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "mean_launch_us": round(dec["mean_launch_us"], 3), "per_layer": dec["layers"]},
        "checkpoint_layout": None if dec_ck is None else {
            "value": round(dec_ck["wbytes"] / (dec_ck["ms_per_step"] * 1e-3) / 1e9, 1),
            "ms_per_step": round(dec_ck["ms_per_step"], 5), "achieved": round(dec_ck["achieved"], 1),
            "frac": round(dec_ck["achieved"] / HBM_PEAK_GBPS, 4), "mean_launch_us": round(dec_ck["mean_launch_us"], 3),
            "per_layer": dec_ck["layers"]},
        "decode_other": dec_other,
        "moe": moe,
        "copy_GBps": round(ceiling, 1),
        "prefill": prefill,
        "bf16": bf16,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
