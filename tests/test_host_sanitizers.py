"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

gptq_api.cpp (argument checks, launch planning, describe strings, workspace and
scratch bookkeeping) is compiled with the host sanitizers and linked with the
library's other objects into tests/host/host_checks.cpp, a driver that calls
the host-only entry points from stdin.  Edge and random arguments (bad bits,
group sizes, shapes at and past the size limits, NULL and misaligned pointers,
every path / wave option, describe buffers down to one byte) must give the same
results as the production library, and the sanitizers must report nothing.
Entry points that launch kernels are called only with arguments their checks
reject, so nothing touches a device.
"""
import ctypes
import os
import random
import shutil
import subprocess

import pytest

import weight_only_bit_gptq_amd as gq
from weight_only_bit_gptq_amd import build_lib
from workload import BENCH_CASES, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "host", "host_checks.cpp")
OTHER_OBJS = ["dequant", "decode", "prefill", "quantize", "ceiling"]


def _objs_ready():
    return all(os.path.exists(os.path.join(build_lib.BUILD, o + ".o")) for o in OTHER_OBJS) and \
        os.path.exists(gq.library_path())


pytestmark = pytest.mark.skipif(not _objs_ready() or not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs the library built (__graft_entry__.build()) and hipcc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    d = tmp_path_factory.mktemp("host_san")
    cc = build_lib.hipcc()
    flags = ["-x", "hip", f"--offload-arch={build_lib.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{build_lib.INCLUDE}", f"-I{build_lib.CSRC}"]
    api = str(d / "gptq_api.o")
    main = str(d / "host_checks.o")
    exe = str(d / "host_checks")
    for src, obj in ((os.path.join(build_lib.CSRC, "gptq_api.cpp"), api), (DRIVER, main)):
        r = subprocess.run([cc, *flags, "-c", src, "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                           text=True)
        assert r.returncode == 0, r.stdout
    objs = [os.path.join(build_lib.BUILD, o + ".o") for o in OTHER_OBJS]
    r = subprocess.run([cc, f"--offload-arch={build_lib.ARCH}", "-Xarch_host", "-fsanitize=address,undefined",
                        "-o", exe, main, api, *objs], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return exe


def run_driver(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                       text=True, env=env, timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    out = r.stdout.splitlines()
    assert len(out) == len(lines), (len(out), len(lines))
    return out


X, QW, QZ, SC, GI, OUT = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000


def gemm_arg_grid(rng):
    """Edge values of every argument plus random combinations."""
    bits_v = [-1, 0, 1, 2, 3, 4, 5, 8, 16]
    gs_v = [-32, 0, 16, 32, 64, 96, 128, 4096]
    mnk = [-1, 0, 1, 4, 16, 17, 32, 48, 96, 1024, 4096, 11008, 1 << 20, (1 << 20) + 32, 1 << 24, (1 << 24) + 1]
    ptrs = [0, 0x10000, 0x10008, 0x10004, 0x10002]
    cases = []
    for bits in bits_v:
        for gs in gs_v:
            cases.append((X, QW, QZ, SC, 0, bits, gs, 1, 1, 4096, 4096, OUT, 0, 0))
    for M in mnk:
        for N in mnk:
            cases.append((X, QW, QZ, SC, 0, 4, 128, 0, M, N, 4096, OUT, 0, 0))
            cases.append((X, QW, QZ, SC, 0, 3, 32, 0, 16, N, M if M > 0 else 32, OUT, 0, 0))
    for i, p in enumerate(ptrs):
        for slot in range(6):
            a = [X, QW, QZ, SC, GI, OUT]
            a[slot] = p
            cases.append((*a, 4, 128, 1, 2, 512, 1024, 0, 0))
    for path in (-1, 0, 1, 2, 3):
        for waves in (-1, 0, 1, 3, 8, 16, 17):
            for M in (1, 16, 17, 2048):
                cases.append((X, QW, QZ, SC, 0, 4, 128, 1, M, 4096, 8192, OUT, path, waves))
    for _ in range(1500):
        bits = rng.choice([2, 3, 4, 8])
        gs = rng.choice([16, 32, 64, 96, 128, 256, 1024])
        K = gs * rng.randint(1, 64) if rng.random() < 0.8 else 32 * rng.randint(1, 4096)
        N = 32 * rng.randint(1, 2048)
        M = rng.choice([0, 1, 2, 3, 4, 7, 8, 15, 16, 17, 40, 128, 1024, 2048, 4096])
        cases.append((X, QW, QZ, SC, GI if rng.random() < 0.3 else 0, bits, gs, rng.randint(0, 1), M, N, K, OUT,
                      rng.choice([0, 0, 0, 1, 2]), rng.choice([0, 0, 0, 1, 2, 4, 8, 11, 16])))
    for c in BENCH_CASES:
        wl = WORKLOADS[c.workload]
        layer = next(l for l in wl.layers if l.name == c.layer)
        cases.append((X, QW, QZ, SC, GI if (wl.act_order and c.entry == "gemm") else 0, wl.bits, wl.group_size,
                      int(wl.is_v2), c.M, layer.N, layer.K, OUT, 0, 0))
    return cases


def fmt(op, a, buflen=None):
    h = lambda v: format(v, "x")
    s = f"{op} {h(a[0])} {h(a[1])} {h(a[2])} {h(a[3])} {h(a[4])} " + " ".join(str(v) for v in a[5:11]) + \
        f" {h(a[11])} {a[12]} {a[13]}"
    return s + f" {256 if buflen is None else buflen}"


def test_host_code_under_sanitizers(driver):
    lib = gq.library()
    rng = random.Random(7)
    grid = gemm_arg_grid(rng)
    lines, want = [], []
    for a in grid:
        nul = lambda v: None if v == 0 else v
        args = (nul(a[0]), nul(a[1]), nul(a[2]), nul(a[3]), nul(a[4]), *a[5:11], nul(a[11]))
        lines.append(fmt("gemm", a))
        want.append(str(lib.gptq_gemm_check(*args)))
        lines.append(fmt("gemm_ex", a))
        code = lib.gptq_gemm_ex_check(*args, a[12], a[13])
        want.append(str(code))
        for op, fn in (("describe", lib.gptq_gemm_describe), ("tiled_describe", lib.gptq_gemm_tiled_describe),
                       ("bf16_describe", lib.gptq_gemm_bf16_describe),
                       ("tiled_bf16_describe", lib.gptq_gemm_tiled_bf16_describe)):
            bl = rng.choice([256, 256, 256, 1, 8, 40, 0, -1])
            lines.append(fmt(op, a, bl))
            buf = ctypes.create_string_buffer(512)
            rc = fn(*args, a[12], a[13], None if bl < 0 else buf, min(bl, 512))
            want.append(f"{rc} {buf.value.decode()}" if bl > 0 else str(rc))
        if code != 0:
            # entry points that launch, with arguments their checks reject
            lines.append(fmt("gemm_call", a))
            want.append(str(code))
            if a[12] == 0 and a[13] == 0:
                lines.append(fmt("noalloc_call", a))
                want.append(str(lib.gptq_gemm_check(*args)))
    for bits in (1, 2, 3, 4, 8):
        for (gs, K, N) in ((128, 4096, 4096), (0, 4096, 4096), (96, 4096, 96), (128, 4096, 48)):
            for (qw, qz, sc, out) in ((QW, QZ, SC, OUT), (0, QZ, SC, OUT), (QW, QZ, SC, 0), (QW + 4, QZ, SC, OUT)):
                lines.append(f"dequant_check {qw:x} {qz:x} {sc:x} 0 {bits} {gs} 1 {N} {K} {out:x}")
                want.append(str(lib.gptq_dequant_check(qw or None, qz or None, sc or None, None, bits, gs, 1, N, K,
                                                        out or None)))
    for bits in (2, 3, 4, 8, 5):
        for (G, N) in ((1, 32), (0, 32), (7, 4128), (4, 48), (1 << 20, 32)):
            for (i, o, c) in ((QW, QZ, 0), (QW, QW, 0), (QW, QW + 4, 0), (QW, QZ, 0x70002)):
                for to_v2 in (0, 1, 2):
                    lines.append(f"convert_check {i:x} {o:x} {bits} {G} {N} {to_v2} {c:x}")
                    want.append(str(lib.gptq_convert_zeros_check(i, o, bits, G, N, to_v2, c or None)))
    for code in range(-12, 2):
        lines.append(f"strerror {code}")
        want.append(lib.gptq_strerror(code).decode())
    # launching entry points whose checks reject: repack (overlap, bits, shape), read ceiling
    lines += ["repack_call 20000 20000 4 4096 4096", "repack_call 20000 30000 5 4096 4096",
              "repack_call 20000 30000 4 48 4096", "repack_call 0 30000 4 4096 4096",
              "ceiling_call 20000 -16 30000", "ceiling_call 20000 17 30000", "ceiling_call 0 16 30000",
              "ceiling_call 20008 16 30000"]
    want += [str(lib.gptq_repack_tiled(QW, QW, 4, 4096, 4096, None)),
             str(lib.gptq_repack_tiled(QW, QZ, 5, 4096, 4096, None)),
             str(lib.gptq_repack_tiled(QW, QZ, 4, 48, 4096, None)),
             str(lib.gptq_repack_tiled(None, QZ, 4, 4096, 4096, None)),
             str(lib.gptq_read_ceiling(QW, -16, QZ, None)), str(lib.gptq_read_ceiling(QW, 17, QZ, None)),
             str(lib.gptq_read_ceiling(None, 16, QZ, None)), str(lib.gptq_read_ceiling(0x20008, 16, QZ, None))]
    assert all(w != "0" for w in want[-8:])
    got = run_driver(driver, lines)
    bad = [(l, w, g) for l, w, g in zip(lines, want, got) if w != g]
    assert not bad, bad[:10]
    assert len(lines) > 8000
