#!/usr/bin/env python3
"""Benchmark of the GPTQ weight-only GEMM on one MI355X.

Metric: "GPTQ W4A16 GEMM: weight GB/s at M=1 and TFLOP/s at M=2048, % of
roofline".  A step is one decode pass over the four Llama-7B-shaped layers
(qkv 4096->12288, o_proj 4096->4096, gate_up 4096->22016, down 11008->4096) at
M=1, 4-bit g128 symmetric GPTQv1, synthetic seeded weights quantized on the
GPU by the library's own quantizer, qweight then re-laid out once into the
tiled layout (gptq_repack_tiled, untimed).  `value` = packed weight bytes
(qweight + qzeros + scales) per step / step time.  Distinct weight copies
(>= 1 GiB in total) are rotated so the 256 MB Infinity Cache cannot serve them.

Every GEMM call timed here is one of workload.BENCH_CASES, the list the GPU
parity tests run (tests/test_gpu_bench_parity.py).  Timing: launches are
captured in HIP graphs (no Python overhead in the timed region) and timed with
HIP events on the stream the graphs replay on; a per-call figure is the median
over 5 replays of a graph of >= 50 launches.  The headline step time is one
replay of a graph of exactly --steps steps, after --warmup eager steps and
--warm-seconds of untimed replays (MI355X raises its clocks over hundreds of
milliseconds of load).

The JSON line also carries:
  roofline      the decode kernel: algorithmic bytes per launch (weights + x +
                y) / its median launch time, against 8 TB/s, and per layer the
                time of gptq_read_ceiling (a plain read of the same bytes) as
                the achievable floor;
  decode_checkpoint, decode_other, moe, prefill, prefill_checkpoint, bf16:
                the other benchmarked calls;
  cpu_baseline  the CPU oracle (numpy, fp64) on a bounded column slice of the
                qkv layer, same unit, dequant and matmul timed apart;
  parity        every timed call's output on sampled 32-column blocks against
                the oracle (run in the same leg as cpu_baseline; a mismatch
                makes the run exit with status 3).

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20]

Counter passes (HBM traffic of the decode kernel, see `--pmc-driver`):
  rocprofv3 --pmc FETCH_SIZE -d D/fetch -o run -f csv -- python3 bench.py --pmc-driver
  rocprofv3 --pmc WRITE_SIZE -d D/write -o run -f csv -- python3 bench.py --pmc-driver
  python3 bench.py --summarize-pmc D/fetch/run_counter_collection.csv D/write/run_counter_collection.csv
The summary goes to profiles/; `roofline.traffic` is read from it while the
decode sources still hash to the value recorded there (null otherwise).

Counter pass (MFMA utilisation of the prefill kernel, see `--pmc-prefill-driver`):
  rocprofv3 --pmc MfmaUtil GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA --kernel-trace -d D/mfma -o run -f csv \\
      -- python3 bench.py --pmc-prefill-driver
  python3 bench.py --summarize-prefill-pmc D/mfma/run_counter_collection.csv D/mfma/run_kernel_trace.csv
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama7b_w4g128_hbm_traffic.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_mlp70b_mfma_util.txt")
DECODE_PMC_FILE = os.path.join(ROOT, "profiles", "decode_all_instructions_and_stalls.txt")
DECODE_PMC_GROUPS = ("decode", "decode_other")
DECODE_TRACE_FILE = os.path.join(ROOT, "profiles", "decode_llama7b_w4g128_kernel_trace.txt")
PREFILL_TRACE_FILE = os.path.join(ROOT, "profiles", "prefill_mlp70b_kernel_trace.txt")
TRACE_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -f csv -d D/trace -o run -- python3 R/bench.py "
             "--steps 50 --warmup 10 --prefill-steps 3 --no-cpu-baseline --no-checkpoint-layout --no-bf16 --no-other "
             "> D/trace_bench.log; python3 R/bench.py --summarize-trace D/trace/run_kernel_stats.csv D/trace_bench.log")
# sources that decide the decode kernel's code and launch shapes
DECODE_SOURCES = ["weight_only_bit_gptq_amd/csrc/decode.hip", "weight_only_bit_gptq_amd/csrc/gptq_device.hpp",
                  "weight_only_bit_gptq_amd/csrc/gptq_kernels.hpp", "weight_only_bit_gptq_amd/csrc/gptq_api.cpp"]
ALL_SOURCES = DECODE_SOURCES + ["weight_only_bit_gptq_amd/csrc/prefill.hip", "weight_only_bit_gptq_amd/csrc/dequant.hip",
                                "weight_only_bit_gptq_amd/csrc/quantize.hip", "weight_only_bit_gptq_amd/csrc/ceiling.hip",
                                "bench.py"]
PMC_COPY_BYTES = 256 << 20      # plain copy of known size that calibrates FETCH_SIZE / WRITE_SIZE

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 (and bf16) MFMA
ROTATE_BYTES = 1 << 30          # rotate >= 1 GiB of distinct weight copies
MIN_LAUNCHES = 50               # launches per timed graph replay
REPS = 5                        # timed replays per figure (median reported)
TOL = 5e-3                      # GEMM parity bar: max|y - y_ref| <= TOL * rms(y_ref)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--prefill-steps", type=int, default=10, help="launches per timed prefill repetition")
    p.add_argument("--warm-seconds", type=float, default=0.5,
                   help="untimed GPU work before each timed region (MI355X raises its clocks over "
                        "hundreds of milliseconds of load; measured without it, prefill reads ~15%% low)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-checkpoint-layout", action="store_true",
                   help="skip the calls on the checkpoint qweight layout (reported beside the tiled ones)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle leg (cpu_baseline and the parity check of the timed outputs)")
    p.add_argument("--no-bf16", action="store_true",
                   help="skip the bfloat16-activation lines (decode layers and 4-bit prefill)")
    p.add_argument("--no-other", action="store_true", help="skip decode_other, small_batch and moe")
    p.add_argument("--cpu-sample-cols", type=int, default=12288,
                   help="columns of the qkv layer the CPU oracle processes (default: all)")
    p.add_argument("--cpu-reps", type=int, default=3, help="at least this many oracle calls on the sample")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="repeat the oracle on the sample until this much time has passed (median reported)")
    p.add_argument("--pmc-driver", action="store_true",
                   help="only launch each decode layer 3 times and a plain copy, for a rocprofv3 --pmc pass")
    p.add_argument("--pmc-decode-driver", action="store_true",
                   help="only launch every benchmarked decode call 3 times, for rocprofv3 --pmc passes")
    p.add_argument("--summarize-decode-pmc", nargs="+", metavar="COUNTER_CSV",
                   help="write the decode instruction / stall summary to profiles/ from --pmc-decode-driver passes")
    p.add_argument("--pmc-prefill-driver", action="store_true",
                   help="only launch each 70B-MLP prefill layer twice, for a rocprofv3 --pmc pass")
    p.add_argument("--summarize-prefill-pmc", nargs=2, metavar=("COUNTER_CSV", "TRACE_CSV"),
                   help="write the prefill MFMA-utilisation summary to profiles/ from a --pmc-prefill-driver pass")
    p.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "BENCH_LOG"),
                   help="write the decode and prefill kernel-trace summaries to profiles/ from a rocprofv3 "
                        "--kernel-trace --stats run of this bench (TRACE_CMD) and that run's output")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the HBM traffic summary from two counter passes (no GPU needed)")
    return p.parse_args()


def sources_hash(paths):
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_sources_hash():
    return sources_hash(DECODE_SOURCES)


def git_head():
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], stdout=subprocess.PIPE,
                           stderr=subprocess.DEVNULL, text=True, timeout=10)
        return r.stdout.strip() or None
    except Exception:
        return None


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


def wl_layer(case):
    from workload import WORKLOADS
    wl = WORKLOADS[case.workload]
    return wl, next(l for l in wl.layers if l.name == case.layer)


def check_cols(N):
    """Output columns the oracle checks: three 32-column blocks (first, middle,
    last), so the oracle can quantize just those columns (columns are
    quantized independently; qzeros packs 32 columns per 32*b/32 words)."""
    mid = (N // 2) // 32 * 32
    return np.unique(np.concatenate([np.arange(0, 32), np.arange(mid, mid + 32), np.arange(N - 32, N)]))


# ---------------------------------------------------------------- timing helpers
def warm(torch, fn, seconds):
    """Untimed calls of fn until `seconds` have passed (clocks settle)."""
    t0 = time.perf_counter()
    while True:
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break


def median_replay_ms(torch, graph, reps=REPS):
    """Median over `reps` replays of a graph, each bracketed by HIP events on
    the stream the replay runs on (torch's current stream)."""
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        e0.record(st)
        graph.replay()
        e1.record(st)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts)), ts


def capture(torch, dev, launches):
    """A HIP graph of the given launch closures (captured on a side stream
    after one eager pass that also allocates any library workspace)."""
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for f in launches:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for f in launches:
            f()
    torch.cuda.synchronize()
    return g


# ---------------------------------------------------------------- one benchmarked call
def prepare(torch, gq, case, dev):
    """The call's inputs on the GPU: seeded draw, quantized by the library's
    quantizer, tiled / sorted at load as the case says, bf16 x and scales for
    bf16 cases.  Returns a dict with a `call(qweight, out)` closure."""
    from workload import draw_workload_layer
    wl, layer = wl_layer(case)
    d = draw_workload_layer(wl, layer, max(wl.Ms), seed=0)
    w = torch.from_numpy(d.W).to(dev)
    gi = None if d.g_idx is None else torch.from_numpy(d.g_idx).to(dev)
    qw, qz, sc = gq.quantize(w, gi, wl.bits, wl.group_size, wl.sym, wl.is_v2)
    del w, d.W
    perm = None
    if case.entry == "gemm_sorted":
        qw, perm = gq.sort_act_order(qw, gi, wl.bits, wl.group_size)
    if case.layout == "tiled":
        qw = gq.repack_tiled(qw, wl.bits)
    x = torch.from_numpy(d.x[:case.M]).to(dev)
    if case.act == "bf16":
        x, sc = x.to(torch.bfloat16), sc.to(torch.bfloat16)
    gi_call = None if case.entry == "gemm_sorted" else gi

    def call(qweight, out):
        if perm is not None:
            gq.gemm_sorted(x, qweight, qz, sc, perm, wl.bits, wl.group_size, wl.is_v2, out=out)
        else:
            gq.gemm(x, qweight, qz, sc, gi_call, wl.bits, wl.group_size, wl.is_v2, out=out)

    desc = gq.describe(x, qw, qz, sc, gi_call, wl.bits, wl.group_size, wl.is_v2)
    if perm is not None:
        desc = "x gathered by perm, then " + desc
    wb = layer_bytes(layer.K, layer.N, wl.bits, wl.group_size) + (4 * layer.K if gi_call is not None else 0)
    alg = wb + 2 * case.M * layer.K + 2 * case.M * layer.N
    return dict(case=case, wl=wl, layer=layer, qweight=qw, x=x, call=call, desc=desc, wbytes=wb, alg=alg,
                act=torch.bfloat16 if case.act == "bf16" else torch.float16)


def rotated_copies(torch, P, nbytes_per_set):
    """[qweight, clone, ...]: enough distinct copies that together they exceed
    ROTATE_BYTES (each call then reads weights no cache holds)."""
    copies = max(2, -(-ROTATE_BYTES // nbytes_per_set))
    return [P["qweight"]] + [P["qweight"].clone() for _ in range(copies - 1)]


def time_decode_call(torch, P, dev, args, sets=None):
    """Median launch time (us) of one decode call over rotated weight copies;
    also returns the output of a launch on the first copy."""
    sets = sets or rotated_copies(torch, P, P["wbytes"])
    out = torch.empty((P["case"].M, P["layer"].N), dtype=P["act"], device=dev)
    n = max(MIN_LAUNCHES, len(sets))
    g = capture(torch, dev, [lambda i=i: P["call"](sets[i % len(sets)], out) for i in range(n)])
    warm(torch, g.replay, args.warm_seconds / 4)
    ms, ts = median_replay_ms(torch, g)
    del g
    P["call"](sets[0], out)
    torch.cuda.synchronize()
    return ms * 1e3 / n, [round(t * 1e3 / n, 3) for t in ts], out


def time_read_ceiling(torch, gq, nbytes, dev, args):
    """Median time (us) of gptq_read_ceiling over `nbytes` (rounded up to 16),
    rotated over distinct buffers like the decode weights."""
    nb = (nbytes + 4095) // 4096 * 4096
    copies = max(2, -(-ROTATE_BYTES // nb))
    buf = torch.ones(copies * nb // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    n = max(MIN_LAUNCHES, copies)
    g = capture(torch, dev, [lambda i=i: gq.read_ceiling(buf[(i % copies) * nb // 4:((i % copies) + 1) * nb // 4],
                                                         (nbytes + 15) // 16 * 16, sink=sink) for i in range(n)])
    warm(torch, g.replay, args.warm_seconds / 4)
    ms, _ = median_replay_ms(torch, g)
    del g, buf
    return ms * 1e3 / n


# ---------------------------------------------------------------- decode step (headline)
def bench_decode_step(torch, gq, args, dev, group, outputs):
    """The four Llama-7B layers as a decode step: per-layer median launch
    times, the step time (one replay of exactly --steps steps) and the read
    ceiling of each layer's bytes."""
    from workload import bench_cases
    cases = bench_cases(group)
    Ps = [prepare(torch, gq, c, dev) for c in cases]
    step_bytes = sum(P["wbytes"] for P in Ps)
    copies = max(2, -(-ROTATE_BYTES // step_bytes))
    sets = [[P["qweight"]] + [P["qweight"].clone() for _ in range(copies - 1)] for P in Ps]
    outs = [torch.empty((P["case"].M, P["layer"].N), dtype=P["act"], device=dev) for P in Ps]

    def step(i):
        for j, P in enumerate(Ps):
            P["call"](sets[j][i % copies], outs[j])

    for i in range(args.warmup):                        # untimed warm-up steps
        step(i)
    torch.cuda.synchronize()
    g_step = capture(torch, dev, [lambda i=i: step(i) for i in range(args.steps)])
    layers = []
    for j, P in enumerate(Ps):
        us, reps, out = time_decode_call(torch, P, dev, args, sets=sets[j])
        outputs[P["case"].key] = out[:, torch.from_numpy(check_cols(P["layer"].N)).to(dev)].float().cpu().numpy()
        layers.append(dict(layer=P["layer"].name, K=P["layer"].K, N=P["layer"].N, kernel=P["desc"],
                           alg_bytes=P["alg"], us=round(us, 3), reps_us=reps,
                           GBps=round(P["alg"] / (us * 1e-6) / 1e9, 1)))
    warm(torch, g_step.replay, args.warm_seconds)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g_step.replay()                                     # exactly args.steps steps
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    del g_step
    mean_us = float(np.mean([l["us"] for l in layers]))
    mean_alg = float(np.mean([l["alg_bytes"] for l in layers]))
    return dict(wl=Ps[0]["wl"], wbytes=step_bytes, copies=copies, ms_per_step=ms_per_step, layers=layers,
                mean_launch_us=mean_us, achieved=mean_alg / (mean_us * 1e-6) / 1e9,
                value=step_bytes / (ms_per_step * 1e-3) / 1e9)


def add_ceilings(torch, gq, args, dev, layers, bits, gs):
    for l in layers:
        wb = layer_bytes(l["K"], l["N"], bits, gs)
        c = time_read_ceiling(torch, gq, wb, dev, args)
        l["read_ceiling_us"] = round(c, 3)
        l["of_ceiling"] = round(c / l["us"], 4)


# ---------------------------------------------------------------- the other decode calls
def bench_decode_other(torch, gq, args, dev, outputs, skip_checkpoint):
    """2-bit g64 (M = 1, 4, 16; tiled), 3-bit act-order M = 16 (rows sorted at
    load, tiled; and the unsorted layer through gptq_gemm with g_idx on the
    checkpoint layout): per-call median launch time and the read ceiling of
    the call's weight bytes."""
    from workload import bench_cases
    res = []
    ceilings = {}
    cur = None
    sets = None
    for case in bench_cases("decode_other"):
        if skip_checkpoint and case.layout == "checkpoint":
            continue
        P = prepare(torch, gq, case, dev)
        key = (case.workload, case.layer, case.layout, case.entry)
        if key != cur:
            sets, cur = None, key
            torch.cuda.empty_cache()
        sets = sets or rotated_copies(torch, P, P["wbytes"])
        us, reps, out = time_decode_call(torch, P, dev, args, sets=sets)
        outputs[case.key] = out[:, torch.from_numpy(check_cols(P["layer"].N)).to(dev)].float().cpu().numpy()
        ck = (P["layer"].K, P["layer"].N, P["wl"].bits, P["wl"].group_size)
        if ck not in ceilings:
            ceilings[ck] = time_read_ceiling(torch, gq, layer_bytes(*ck), dev, args)
        res.append({"workload": case.workload, "layer": f"{case.layer} {P['layer'].K}->{P['layer'].N}", "M": case.M,
                    "layout": case.layout, "entry": case.entry, "kernel": P["desc"], "us": round(us, 3),
                    "reps_us": reps, "GBps": round(P["alg"] / (us * 1e-6) / 1e9, 1),
                    "frac": round(P["alg"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "read_ceiling_us": round(ceilings[ck], 3), "of_ceiling": round(ceilings[ck] / us, 4)})
        del P
    return res


def bench_small_batch(torch, gq, args, dev, outputs):
    """The Llama-7B layers at M = 17, 64, 128, 512 (tiled 4-bit) through
    gptq_gemm's automatic plan (prefill tiles of 32-128 rows, K split over
    workgroups when the grid is small): per-call median launch time over
    rotated weight copies, weight GB/s, TFLOP/s and the fraction of the
    binding roofline (HBM for the bytes, fp16 MFMA for the flops)."""
    from workload import bench_cases
    res = []
    cur = sets = None
    for case in bench_cases("small_batch"):
        P = prepare(torch, gq, case, dev)
        if case.layer != cur:
            sets, cur = None, case.layer
            torch.cuda.empty_cache()
        sets = sets or rotated_copies(torch, P, P["wbytes"])
        us, reps, out = time_decode_call(torch, P, dev, args, sets=sets)
        outputs[case.key] = out[:, torch.from_numpy(check_cols(P["layer"].N)).to(dev)].float().cpu().numpy()
        K, N = P["layer"].K, P["layer"].N
        gbps = P["alg"] / (us * 1e-6) / 1e9
        tf = 2.0 * case.M * K * N / (us * 1e-6) / 1e12
        # the binding roofline at these sizes: the algorithmic bytes (weights,
        # x, y) against HBM, or the flops against the fp16 MFMA peak
        res.append({"workload": case.workload, "layer": f"{case.layer} {K}->{N}", "M": case.M,
                    "kernel": P["desc"], "us": round(us, 3), "reps_us": reps,
                    "weight_GBps": round(P["wbytes"] / (us * 1e-6) / 1e9, 1), "TFLOPs": round(tf, 1),
                    "roofline_frac": round(max(gbps / HBM_PEAK_GBPS, tf / MFMA_F16_PEAK_TFLOPS), 4)})
        del P
    return res


def bench_moe(torch, gq, args, dev, tokens):
    """Grouped GEMM (gptq_moe_gemm) on a Mixtral-class expert layer: 8 experts
    4096 -> 14336, 4-bit g128 sym v1, `tokens` tokens routed top-2 (seeded),
    weight copies rotated past the Infinity Cache.  16 tokens (at most 16 rows
    per expert: the decode kernel) report weight GB/s over the experts that
    received tokens (all of them read once per launch); 2048 tokens (hundreds
    of rows per expert: the grouped prefill kernel) report TFLOP/s as well."""
    E, K, N, bits, gs = 8, 4096, 14336, 4, 128
    rng = np.random.default_rng(0)
    picks = np.array([rng.choice(E, size=2, replace=False) for _ in range(tokens)]).ravel()
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
    n = max(MIN_LAUNCHES, copies) if mt <= 16 else copies
    g = capture(torch, dev, [lambda i=i: gq.moe_gemm(x, *sets[i % copies], None, offsets, mt, bits, gs, False, out=out)
                             for i in range(n)])
    warm(torch, g.replay, args.warm_seconds)
    ms, _ = median_replay_ms(torch, g)
    us = ms * 1e3 / n
    del g, sets, base
    torch.cuda.empty_cache()
    res = {"workload": "mixtral_expert_w1_w4g128", "experts": E, "K": K, "N": N, "tokens": tokens, "top_k": 2,
           "active_experts": active, "max_rows_per_expert": mt,
           "kernel": "decode (blocks of 16 rows)" if mt <= 16 else "prefill (128-row tiles per expert)",
           "us": round(us, 2), "weight_GBps": round(wbytes / (us * 1e-6) / 1e9, 1),
           "frac": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    if mt <= 16:
        ceil_us = time_read_ceiling(torch, gq, wbytes, dev, args)
        res.update(read_ceiling_us=round(ceil_us, 2), of_ceiling=round(ceil_us / us, 4))
    else:
        tflops = 2.0 * T * K * N / (us * 1e-6) / 1e12
        res.update(TFLOPs=round(tflops, 1), mfma_frac=round(tflops / MFMA_F16_PEAK_TFLOPS, 4))
    return res


# ---------------------------------------------------------------- prefill
def bench_prefill(torch, gq, args, dev, group, outputs):
    """Prefill GEMM (M = 2048) timing per call: median over 5 repetitions of
    --prefill-steps launches each; for the fp16 4-bit tiled calls the vendor
    dense GEMM in the same activation type on the same shape, as context."""
    from workload import bench_cases
    res = []
    for case in bench_cases(group):
        P = prepare(torch, gq, case, dev)
        layer, wl = P["layer"], P["wl"]
        out = torch.empty((case.M, layer.N), dtype=P["act"], device=dev)
        run = lambda: P["call"](P["qweight"], out)
        warm(torch, run, args.warm_seconds)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(REPS):
            e0.record()
            for _ in range(args.prefill_steps):
                run()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / args.prefill_steps)
        ms = float(np.median(ts))
        outputs[case.key] = out[:, torch.from_numpy(check_cols(layer.N)).to(dev)].float().cpu().numpy()
        flops = 2.0 * case.M * layer.K * layer.N
        tf = flops / (ms * 1e-3) / 1e12
        row = {"workload": case.workload, "layer": layer.name, "M": case.M, "K": layer.K, "N": layer.N,
               "bits": wl.bits, "qweight_layout": case.layout, "kernel": P["desc"], "ms": round(ms, 4),
               "reps_ms": [round(t, 4) for t in ts], "TFLOPs": round(tf, 1),
               "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
        if wl.bits == 4 and case.layout == "tiled" or case.act == "bf16":
            W = torch.randn((layer.K, layer.N), dtype=P["act"], device=dev)
            dense = lambda: torch.matmul(P["x"], W, out=out)
            warm(torch, dense, args.warm_seconds)
            dts = []
            for _ in range(REPS):
                e0.record()
                for _ in range(args.prefill_steps):
                    dense()
                e1.record()
                torch.cuda.synchronize()
                dts.append(e0.elapsed_time(e1) / args.prefill_steps)
            key = "dense_bf16_matmul_TFLOPs" if case.act == "bf16" else "dense_fp16_matmul_TFLOPs"
            row[key] = round(flops / (float(np.median(dts)) * 1e-3) / 1e12, 1)
            del W
        res.append(row)
        del P, out
        torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- oracle leg
def cpu_baseline(args):
    """The oracle (dequant from packed arrays + fp64 matmul) on a column slice
    of the qkv layer, quantized by the oracle itself from the same draw;
    median of --cpu-reps calls, dequant and matmul timed apart."""
    import oracle
    from workload import WORKLOADS, draw_workload_layer
    wl = WORKLOADS["llama7b_decode_w4g128"]
    layer = wl.layers[0]
    d = draw_workload_layer(wl, layer, 1, seed=0)
    ncols = min(args.cpu_sample_cols, layer.N)
    W = np.ascontiguousarray(d.W[:, :ncols])
    L = oracle.quantize_layer(W, wl.bits, wl.group_size, wl.sym, wl.is_v2)
    t_dq, t_mm = [], []
    t_start = time.perf_counter()
    while len(t_dq) < max(1, args.cpu_reps) or time.perf_counter() - t_start < args.cpu_seconds:
        t0 = time.perf_counter()
        Wh = oracle.dequant_ref(L.qweight, L.qzeros, L.scales, None, wl.bits, wl.group_size, wl.is_v2,
                                layer.K, ncols)
        t1 = time.perf_counter()
        oracle.gemm_ref(d.x, Wh)
        t2 = time.perf_counter()
        t_dq.append(t1 - t0)
        t_mm.append(t2 - t1)
    sec = float(np.median(np.array(t_dq) + np.array(t_mm)))
    gbps = layer_bytes(layer.K, ncols, wl.bits, wl.group_size) / sec / 1e9
    blas = 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": blas, "kind": "oracle",
            "cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas_threads": blas,
            "dequant_s": round(float(np.median(t_dq)), 3), "matmul_s": round(float(np.median(t_mm)), 3),
            "sample": f"qkv layer K={layer.K}, first {ncols} of {layer.N} columns, M=1; median of "
                      f"{len(t_dq)} oracle calls of {sec:.2f} s (numpy fp64 dequant, single-threaded: "
                      f"{np.median(t_dq):.2f} s; fp64 matmul through BLAS on up to {blas} threads: "
                      f"{np.median(t_mm):.3f} s)"}


def parity_check(outputs):
    """Every timed call's output on its check columns against the oracle: the
    oracle quantizes only those columns of the same seeded draw (columns are
    independent) and runs its dequant + matmul."""
    import oracle
    import torch
    from workload import BENCH_CASES, draw_workload_layer
    draws = {}
    res = []
    for case in BENCH_CASES:
        if case.key not in outputs:
            continue
        wl, layer = wl_layer(case)
        cols = check_cols(layer.N)
        # the draw depends on the shape and the recipe's random parts only (the
        # 4- and 8-bit 70B-MLP workloads share it)
        dk = (layer.K, layer.N, max(wl.Ms), wl.sigma, wl.outlier_rate, wl.outlier_mult, wl.act_order,
              wl.group_size if wl.act_order else 0)
        if dk not in draws:
            d = draw_workload_layer(wl, layer, max(wl.Ms), seed=0)
            draws[dk] = (np.ascontiguousarray(d.W[:, cols]), d.x, d.g_idx)
            del d
        Wc, x, g_idx = draws[dk]
        L = oracle.quantize_layer(Wc, wl.bits, wl.group_size, wl.sym, wl.is_v2, g_idx)
        xm, sc = x[:case.M], L.scales
        if case.act == "bf16":
            bf = lambda a: torch.from_numpy(np.ascontiguousarray(a.astype(np.float32))).to(torch.bfloat16).to(
                torch.float64).numpy()
            xm, sc = bf(xm), bf(sc)
        ref = oracle.gptq_gemm_ref(xm, L.qweight, L.qzeros, sc, L.g_idx, wl.bits, wl.group_size, wl.is_v2,
                                   layer.K, len(cols), act=case.act)
        y = outputs[case.key].astype(np.float64)
        rms = float(np.sqrt(np.mean(ref ** 2)))
        bound = TOL * rms + (2.0 ** -8 * np.abs(ref) if case.act == "bf16" else 0.0)
        err = np.abs(y - ref)
        ok = bool(np.isfinite(y).all() and (err <= bound).all())
        res.append({"case": case.key, "cols": int(len(cols)), "max_err_over_rms": round(float(err.max()) / rms, 6),
                    "ok": ok})
    return res


# ---------------------------------------------------------------- counter drivers / summaries
def pmc_driver(torch, gq, dev):
    """Each decode layer 3 times (distinct weight copies, so no launch finds its
    weights in L2), then a plain copy of PMC_COPY_BYTES; no timing."""
    from workload import bench_cases
    for case in bench_cases("decode"):
        P = prepare(torch, gq, case, dev)
        out = torch.empty((1, P["layer"].N), dtype=torch.float16, device=dev)
        copies = [P["qweight"].clone() for _ in range(3)]
        torch.cuda.synchronize()
        for qw in copies:
            P["call"](qw, out)
        torch.cuda.synchronize()
        print(f"{case.layer}: {P['desc']}", flush=True)
        del P, copies
    a = torch.ones(PMC_COPY_BYTES // 2, dtype=torch.float16, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("pmc driver done", flush=True)


def pmc_decode_driver(torch, gq, dev):
    """Every benchmarked decode call (groups DECODE_PMC_GROUPS) launched 3
    times on distinct weight copies; one line per call names it."""
    from workload import bench_cases
    for group in DECODE_PMC_GROUPS:
        for case in bench_cases(group):
            P = prepare(torch, gq, case, dev)
            out = torch.empty((case.M, P["layer"].N), dtype=P["act"], device=dev)
            copies = [P["qweight"].clone() for _ in range(3)]
            torch.cuda.synchronize()
            for qw in copies:
                P["call"](qw, out)
            torch.cuda.synchronize()
            print(f"case {case.key}: {P['desc']}", flush=True)
            del P, copies
            torch.cuda.empty_cache()
    print("pmc decode driver done", flush=True)


def summarize_decode_pmc(paths):
    """Per benchmarked decode call: the counters of its 3 launches (mean), from
    one or more --pmc-decode-driver passes, with per-weight instruction counts
    and stall fractions derived where the counters are present."""
    from workload import bench_cases
    cases = [c for g in DECODE_PMC_GROUPS for c in bench_cases(g)]
    per_pass = []
    for path in paths:
        disp = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if "decode_kernel" not in r["Kernel_Name"] and "decode_bf16" not in r["Kernel_Name"]:
                    continue
                d = disp.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ids = sorted(disp)
        if len(ids) != 3 * len(cases):
            raise SystemExit(f"{path}: expected {3 * len(cases)} decode dispatches, got {len(ids)}")
        per_pass.append([disp[i] for i in ids])
    rows = []
    for k, case in enumerate(cases):
        wl, layer = wl_layer(case)
        vals = {"kernel": per_pass[0][3 * k]["kernel"]}
        for launches in per_pass:
            for name in launches[3 * k]:
                if name != "kernel":
                    vals[name] = float(np.mean([launches[3 * k + i][name] for i in range(3)]))
        elems = layer.K * layer.N
        d = {"case": case.key, "kernel": vals["kernel"]}
        for name in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU"):
            if name in vals:
                d[name.replace("SQ_INSTS_", "").lower() + "_lane_per_weight"] = round(64 * vals[name] / elems, 3)
        if "SQ_WAVE_CYCLES" in vals and vals["SQ_WAVE_CYCLES"] > 0:
            for name in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                         "SQ_ACTIVE_INST_VMEM", "SQ_BUSY_CYCLES"):
                if name in vals:
                    d[name.lower() + "_over_wave_cycles"] = round(vals[name] / vals["SQ_WAVE_CYCLES"], 3)
        if "SQ_LDS_BANK_CONFLICT" in vals and vals.get("SQ_INSTS_LDS", 0) > 0:
            d["lds_bank_conflict_cycles_per_lds_inst"] = round(vals["SQ_LDS_BANK_CONFLICT"] / vals["SQ_INSTS_LDS"], 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
            d["mfma_busy_over_gpu_cycles_x_simds"] = round(
                vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (vals["GRBM_GUI_ACTIVE"] / MI355X_XCDS * 1024), 4)
        # L2 side: bytes the L2 served to the CUs (32-byte sectors) over the
        # call's weight bytes (qweight + qzeros + scales): what x and the
        # tables add on top of one read of the weights, re-reads included
        wbytes = layer_bytes(layer.K, layer.N, wl.bits, wl.group_size)
        if "TCC_READ_SECTORS_sum" in vals:
            d["l2_read_bytes_over_weight_bytes"] = round(32 * vals["TCC_READ_SECTORS_sum"] / wbytes, 3)
        if "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals and vals["TCC_HIT_sum"] + vals["TCC_MISS_sum"] > 0:
            d["l2_hit_rate"] = round(vals["TCC_HIT_sum"] / (vals["TCC_HIT_sum"] + vals["TCC_MISS_sum"]), 3)
        if "TCP_TCC_READ_REQ_sum" in vals:
            d["l1_to_l2_read_requests_per_kib_of_weights"] = round(vals["TCP_TCC_READ_REQ_sum"] / (wbytes / 1024), 2)
        d["raw"] = {n: round(v, 1) for n, v in vals.items() if n != "kernel"}
        rows.append(d)
    lines = [
        "# Instruction mix and stalls of every benchmarked decode call (MI355X), rocprofv3 counters",
        "# summed over the chip, mean of 3 launches on distinct weight copies.",
        "# Commands (from /tmp with TMPDIR=/tmp; R = repository root), one pass per counter set:",
        "#   rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
        "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM -d D/p1 -o run -f csv -- python3 R/bench.py --pmc-decode-driver",
        "#   rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_MFMA SQ_INSTS_VMEM_RD SQ_INSTS_SALU "
        "SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -d D/p2 -o run -f csv -- python3 R/bench.py "
        "--pmc-decode-driver",
        "#   rocprofv3 --pmc TCC_READ_SECTORS_sum TCC_HIT_sum TCC_MISS_sum TCP_TCC_READ_REQ_sum -d D/p3 -o run -f csv "
        "-- python3 R/bench.py --pmc-decode-driver",
        "#   python3 R/bench.py --summarize-decode-pmc D/p1/run_counter_collection.csv D/p2/run_counter_collection.csv "
        "D/p3/run_counter_collection.csv",
        "# x_lane_per_weight = 64 * instructions / (K * N): lane-instructions per weight element.",
        "# *_over_wave_cycles: cycles waves spent waiting / issuing, over all wave cycles.",
        "# l2_read_bytes_over_weight_bytes = 32 * TCC_READ_SECTORS / (qweight + qzeros + scales bytes): what the L2",
        "# served the CUs, over one read of the weights (x and re-reads on top); l2_hit_rate = hits / (hits + misses).",
    ]
    for d in rows:
        lines.append(d["case"] + " | " + d["kernel"].split("(")[0].replace("void ", "") + " | " +
                     ", ".join(f"{k}={v}" for k, v in d.items() if k not in ("case", "kernel", "raw")))
    lines.append("json: " + json.dumps({"sources_sha256": decode_sources_hash(), "rows": rows}))
    os.makedirs(os.path.dirname(DECODE_PMC_FILE), exist_ok=True)
    with open(DECODE_PMC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


PREFILL_WORKLOADS = ("mlp70b_prefill_w4g128", "mlp70b_prefill_w8g128")
MI355X_XCDS = 8


def pmc_prefill_driver(torch, gq, dev):
    """Each 70B-MLP prefill layer (M = 2048, tiled layout) twice on its own weights; no timing."""
    from workload import bench_cases
    for case in bench_cases("prefill"):
        P = prepare(torch, gq, case, dev)
        out = torch.empty((case.M, P["layer"].N), dtype=torch.float16, device=dev)
        torch.cuda.synchronize()
        for _ in range(2):
            P["call"](P["qweight"], out)
        torch.cuda.synchronize()
        print(f"{case.workload} {case.layer}: {P['desc']}", flush=True)
        del P, out
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
            if "gptq::prefill_" in r["Kernel_Name"]:
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


def summarize_trace(stats_csv, bench_log):
    """Kernel durations of the decode and prefill launches from rocprofv3's
    kernel statistics, next to the same run's HIP-event figures."""
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3))
    with open(bench_log) as f:
        bench = json.loads([l for l in f if l.startswith("{")][-1])
    avg = {n: a for n, c, a, mi, ma in rows}

    def table(filt):
        out = ["kernel | calls | average us | min us | max us"]
        out += [f"{n} | {c} | {a:.2f} | {mi:.2f} | {ma:.2f}" for n, c, a, mi, ma in rows if filt(n)]
        return out

    def full(desc):
        return "void " + desc.split(" grid=")[0] + "(gptq::GemmArgs)"

    rf = bench["roofline"]
    dec = ["# Kernel durations of the decode kernel, Llama-7B-shaped decode layers (M=1, 4-bit, group 128,",
           "# symmetric, GPTQv1, qweight in the tiled layout), one MI355X; rocprofv3 kernel-trace statistics.",
           "# Command (R = repository root, D = output folder): " + TRACE_CMD,
           f"# sources_sha256 {decode_sources_hash()}", "#"]
    dec += table(lambda n: "gptq::decode_kernel" in n)
    dec += ["", "# Same layers timed by bench.py in the profiled run (HIP events on the launch stream; several",
            "# layers share an instantiation, whose rocprofv3 average mixes them):",
            "layer | kernel | bench us | rocprofv3 average us of its instantiation | read ceiling us"]
    for l in rf["per_layer"]:
        dec.append(f"{l['layer']} | {l['kernel']} | {l['us']:.2f} | {avg.get(full(l['kernel']), float('nan')):.2f} | "
                   f"{l.get('read_ceiling_us', float('nan'))}")
    mean_r = float(np.mean([avg.get(full(l["kernel"]), float("nan")) for l in rf["per_layer"]]))
    mean_b = float(np.mean([l["us"] for l in rf["per_layer"]]))
    dec.append(f"# four layers: rocprofv3 mean of the instantiations {mean_r:.3f} us, bench mean {mean_b:.3f} us; "
               f"achieved {rf['achieved']} GB/s ({100 * rf['frac']:.1f}% of 8 TB/s), step value {bench['value']} GB/s")
    with open(DECODE_TRACE_FILE, "w") as f:
        f.write("\n".join(dec) + "\n")
    pre = ["# Kernel durations of the prefill kernels, 70B-MLP shapes at M=2048 (4-bit g128 sym v1 and 8-bit g128",
           "# asym v2; K=8192->N=28672 and K=28672->N=8192, tiled layout), one MI355X; rocprofv3 kernel-trace",
           "# statistics (no warm-up of the clocks under the profiler: the HIP-event figures below had one).",
           "# Command (R = repository root, D = output folder): " + TRACE_CMD, "#"]
    pre += table(lambda n: "gptq::prefill_" in n)
    pre += ["", "# bench.py (profiled run, HIP events): " + "; ".join(
        f"{p['workload']} {p['layer']} {p['kernel'].split(' grid')[0]} {p['ms']} ms {p['TFLOPs']} TFLOP/s "
        f"({100 * p['frac']:.1f}% of 2.5 PFLOP/s)" for p in bench.get("prefill") or [])]
    with open(PREFILL_TRACE_FILE, "w") as f:
        f.write("\n".join(pre) + "\n")
    print("\n".join(dec))
    print("\n".join(pre))


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


# ---------------------------------------------------------------- main
def decode_summary(d):
    return {"value": round(d["value"], 1), "ms_per_step": round(d["ms_per_step"], 5), "achieved": round(d["achieved"], 1),
            "frac": round(d["achieved"] / HBM_PEAK_GBPS, 4), "mean_launch_us": round(d["mean_launch_us"], 3),
            "per_layer": d["layers"]}


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_prefill_pmc:
        summarize_prefill_pmc(*args.summarize_prefill_pmc)
        return
    if args.summarize_decode_pmc:
        summarize_decode_pmc(args.summarize_decode_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
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
    if args.pmc_decode_driver:
        pmc_decode_driver(torch, gq, dev)
        return

    outputs = {}
    dec = bench_decode_step(torch, gq, args, dev, "decode", outputs)
    wl = dec["wl"]
    add_ceilings(torch, gq, args, dev, dec["layers"], wl.bits, wl.group_size)
    print(f"# decode (tiled): {dec['ms_per_step'] * 1e3:.2f} us/step, layers: {dec['layers']}", file=sys.stderr,
          flush=True)
    torch.cuda.empty_cache()
    dec_ck = None
    if not args.no_checkpoint_layout:
        dec_ck = bench_decode_step(torch, gq, args, dev, "decode_checkpoint", outputs)
        print(f"# decode (checkpoint layout): {dec_ck['ms_per_step'] * 1e3:.2f} us/step, layers: {dec_ck['layers']}",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    dec_other = small = moe = moe_prefill = None
    if not args.no_other:
        dec_other = bench_decode_other(torch, gq, args, dev, outputs, args.no_checkpoint_layout)
        print(f"# other decode calls: {dec_other}", file=sys.stderr, flush=True)
        small = bench_small_batch(torch, gq, args, dev, outputs)
        print(f"# small batches: {small}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        moe = bench_moe(torch, gq, args, dev, 16)
        print(f"# moe: {moe}", file=sys.stderr, flush=True)
        moe_prefill = bench_moe(torch, gq, args, dev, 2048)
        print(f"# moe (prefill batch): {moe_prefill}", file=sys.stderr, flush=True)
    prefill = prefill_ck = None
    if not args.no_prefill:
        prefill = bench_prefill(torch, gq, args, dev, "prefill", outputs)
        print(f"# prefill: {prefill}", file=sys.stderr, flush=True)
        if not args.no_checkpoint_layout:
            prefill_ck = bench_prefill(torch, gq, args, dev, "prefill_checkpoint", outputs)
            print(f"# prefill (checkpoint layout): {prefill_ck}", file=sys.stderr, flush=True)
    bf16 = None
    if not args.no_bf16:
        torch.cuda.empty_cache()
        dec_bf = bench_decode_step(torch, gq, args, dev, "bf16_decode", outputs)
        dec_bft = bench_decode_step(torch, gq, args, dev, "bf16_decode_tiled", outputs)
        bf16 = {"decode": {"workload": dec_bf["wl"].name + " with bf16 x and scales (checkpoint layout)",
                           **decode_summary(dec_bf)},
                "decode_tiled": {"workload": dec_bft["wl"].name + " with bf16 x and scales (tiled layout)",
                                 **decode_summary(dec_bft)},
                "prefill": None if args.no_prefill else bench_prefill(torch, gq, args, dev, "bf16_prefill", outputs)}
        print(f"# bf16: {bf16}", file=sys.stderr, flush=True)
    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args)
        parity = parity_check(outputs)
        print(f"# parity: {parity}", file=sys.stderr, flush=True)

    traffic = read_traffic()
    traffic_bytes = None
    if traffic is not None:
        by_layer = {t["layer"]: t for t in traffic["layers"]}
        if all(l["layer"] in by_layer for l in dec["layers"]):
            for l in dec["layers"]:
                l["traffic_bytes"] = by_layer[l["layer"]]["traffic_bytes"]
            traffic_bytes = int(np.mean([l["traffic_bytes"] for l in dec["layers"]]))
    ceil_sum = sum(l["read_ceiling_us"] for l in dec["layers"])
    line = {
        "metric": "GPTQ W4A16 GEMM: weight GB/s at M=1 and TFLOP/s at M=2048, % of roofline",
        "value": round(dec["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
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
                               "mean algorithmic bytes per launch / mean of the per-layer median launch times; "
                               "traffic = mean HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "mean_launch_us": round(dec["mean_launch_us"], 3),
                     "read_ceiling_step_us": round(ceil_sum, 3),
                     "step_of_read_ceiling": round(ceil_sum / (dec["ms_per_step"] * 1e3), 4),
                     "per_layer": dec["layers"]},
        "decode_checkpoint": None if dec_ck is None else decode_summary(dec_ck),
        "decode_other": dec_other,
        "small_batch": small,
        "moe": moe,
        "moe_prefill": moe_prefill,
        "prefill": prefill,
        "prefill_checkpoint": prefill_ck,
        "bf16": bf16,
        "cpu_baseline": cpu,
        "parity": parity,
        "context": {"pages_kernel_figure": "page 'GPTQ quantization principles and engineering practice', section "
                                           "2.2: a per-column-packed GPTQ kernel ran 17% faster than a block-packed "
                                           "AWQ kernel on an NVIDIA A10 (shapes not given); another machine and "
                                           "metric, not comparable, so vs_baseline stays null",
                    "sources_sha16": sources_hash(ALL_SOURCES), "git": git_head()},
    }
    print(json.dumps(line), flush=True)
    if parity is not None and not all(p["ok"] for p in parity):
        print("parity check failed: " + ", ".join(p["case"] for p in parity if not p["ok"]), file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
