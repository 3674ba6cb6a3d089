"""The benchmark times only calls the GPU parity tests run (no GPU needed).

bench.py draws every GEMM call it times from workload.BENCH_CASES (by group),
and tests/test_gpu_bench_parity.py runs each of those cases through the same
binding call.  This checks both ends of that contract on the CPU, and that the
kernel instantiation and launch shape of every case (gptq_gemm_describe, pure
host code) is one the parity test therefore exercises on the same layout.
"""
import ctypes
import os
import re

import pytest

import weight_only_bit_gptq_amd as gq
from workload import BENCH_CASES, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

needs_lib = pytest.mark.skipif(not os.path.exists(gq.library_path()),
                               reason="libgptq.so not built (run __graft_entry__.build())")


def bench_groups_used():
    src = open(os.path.join(ROOT, "bench.py")).read()
    return set(re.findall(r'bench_cases\("([a-z0-9_]+)"\)', src)) | \
        set(re.findall(r'bench_(?:decode_step|prefill)\(torch, gq, args, dev, "([a-z0-9_]+)"', src))


def test_bench_draws_every_call_from_the_case_list():
    used = bench_groups_used()
    groups = {c.group for c in BENCH_CASES}
    assert used == groups, (used, groups)
    src = open(os.path.join(ROOT, "bench.py")).read()
    # the GEMM entry points are called only inside prepare()'s closure and the MoE line
    body = src[src.index("# ---------------------------------------------------------------- main"):]
    assert "gq.gemm(" not in body and "gq.gemm_sorted(" not in body


def test_gpu_parity_runs_every_bench_case():
    src = open(os.path.join(ROOT, "tests", "test_gpu_bench_parity.py")).read()
    assert '@pytest.mark.parametrize("case", BENCH_CASES, ids=[c.key for c in BENCH_CASES])' in src
    assert "def test_bench_case(dev, case):" in src
    keys = [c.key for c in BENCH_CASES]
    assert len(keys) == len(set(keys))


# fake, suitably aligned addresses: describe never dereferences them
X, QW, QZ, SC, GI, OUT = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000


def describe_case(lib, case):
    wl = WORKLOADS[case.workload]
    layer = next(l for l in wl.layers if l.name == case.layer)
    gi = GI if (wl.act_order and case.entry == "gemm") else None
    buf = ctypes.create_string_buffer(256)
    if case.act == "bf16":
        fn = lib.gptq_gemm_tiled_bf16_describe if case.layout == "tiled" else lib.gptq_gemm_bf16_describe
    else:
        fn = lib.gptq_gemm_tiled_describe if case.layout == "tiled" else lib.gptq_gemm_describe
    code = fn(X, QW, QZ, SC, gi, wl.bits, wl.group_size, int(wl.is_v2), case.M, layer.N, layer.K, OUT, 0, 0,
              buf, 256)
    assert code == 0, (case.key, code)
    return buf.value.decode()


@needs_lib
def test_describe_every_bench_case():
    lib = gq.library()
    seen = {}
    for case in BENCH_CASES:
        d = describe_case(lib, case)
        if case.M <= 16:
            assert d.startswith("gptq::decode"), (case.key, d)
        else:   # the prefill kernel, or (small layers, per-element layers) the decode kernel over row blocks
            assert d.startswith("gptq::prefill") or (d.startswith("gptq::decode") and "row_blocks=" in d), (case.key, d)
        if case.act == "bf16":
            assert "bf16" in d, (case.key, d)
        seen.setdefault(d.split(" grid=")[0], []).append(case.key)
    # the headline's four layers and the 2-bit multi-row calls use the fast path
    for case in BENCH_CASES:
        if case.group in ("decode", "decode_checkpoint") or case.workload == "lowbit_decode_w2g64":
            assert "<%d, false," % WORKLOADS[case.workload].bits in describe_case(lib, case), case.key
    assert seen
