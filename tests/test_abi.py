"""C-ABI checks that need no GPU: the library loads, exports every function
include/gptq.h declares, and its argument checks return the documented codes
(the *_check entry points are pure host code and touch no device)."""
import ctypes
import os
import re

import pytest

import weight_only_bit_gptq_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")

needs_lib = pytest.mark.skipif(not os.path.exists(gq.library_path()),
                               reason="libgptq.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"GPTQ_API\s+[A-Za-z_][A-Za-z0-9_\s\*]*?\b(gptq_[a-z0-9_]+)\s*\(", text)


def declared_status():
    text = open(HEADER).read()
    return {int(v): k for k, v in re.findall(r"\b(GPTQ_[A-Z_]+)\s*=\s*(-?\d+)", text)}


def test_header_declares_api():
    names = declared_functions()
    for f in ("gptq_gemm", "gptq_gemm_ex", "gptq_dequant", "gptq_gemm_check", "gptq_gemm_ex_check",
              "gptq_gemm_describe", "gptq_dequant_check", "gptq_convert_zeros", "gptq_convert_zeros_check",
              "gptq_repack_tiled", "gptq_unrepack_tiled", "gptq_gemm_tiled", "gptq_gemm_tiled_ex",
              "gptq_gemm_tiled_describe", "gptq_moe_gemm", "gptq_moe_gemm_ex", "gptq_sort_act_order", "gptq_gemm_sorted",
              "gptq_gemm_bf16", "gptq_gemm_bf16_ex", "gptq_gemm_bf16_describe", "gptq_dequant_bf16",
              "gptq_gemm_tiled_bf16", "gptq_gemm_tiled_bf16_ex", "gptq_gemm_tiled_bf16_describe",
              "gptq_strerror", "gptq_release", "gptq_abi_version"):
        assert f in names
    assert declared_status() == gq.STATUS


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gq.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert gq.library().gptq_abi_version() == 1


@needs_lib
def test_strerror_covers_every_code():
    lib = gq.library()
    for code in gq.STATUS:
        assert lib.gptq_strerror(code).decode()
    assert lib.gptq_strerror(12345).decode() == "unknown error"


# fake, suitably aligned addresses: the check functions never dereference them
X, QW, QZ, SC, GI, OUT = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000


def gemm_check(x=X, qw=QW, qz=QZ, sc=SC, gi=None, bits=4, gs=128, v2=1, M=1, N=4096, K=4096, out=OUT):
    return gq.library().gptq_gemm_check(x, qw, qz, sc, gi, bits, gs, v2, M, N, K, out)


@needs_lib
def test_gemm_check_codes():
    assert gemm_check() == 0
    assert gemm_check(gi=GI) == 0
    assert gemm_check(M=0, x=None, out=None) == 0
    assert gemm_check(x=None) == -1
    assert gemm_check(qw=None) == -1
    assert gemm_check(qz=None) == -1
    assert gemm_check(sc=None) == -1
    assert gemm_check(out=None) == -1
    for b in (0, 1, 5, 6, 7, 16):
        assert gemm_check(bits=b) == -2
    assert gemm_check(M=-1) == -3
    assert gemm_check(N=0) == -3
    assert gemm_check(K=0) == -3
    assert gemm_check(N=48) == -3
    assert gemm_check(K=4112, gs=16) == -3
    assert gemm_check(K=1 << 21, gs=128) == -3
    assert gemm_check(M=1 << 20, K=4096) == -3       # M*K >= 2^31
    assert gemm_check(gs=0) == -4
    assert gemm_check(gs=-128) == -4
    assert gemm_check(gs=96) == -4                    # 4096 % 96 != 0
    assert gemm_check(x=X + 8) == -5
    assert gemm_check(qw=QW + 4) == -5
    assert gemm_check(out=OUT + 2) == -5
    assert gemm_check(sc=SC + 4) == -5
    assert gemm_check(qz=QZ + 2) == -5
    assert gemm_check(gi=GI + 2) == -5
    assert gemm_check(gi=GI + 4) == -5
    assert gemm_check(v2=2) == -9
    assert gemm_check(bits=3, N=32, K=96, gs=32) == 0


@needs_lib
def test_dequant_check_codes():
    lib = gq.library()
    ok = lambda **kw: lib.gptq_dequant_check(kw.get("qw", QW), kw.get("qz", QZ), kw.get("sc", SC),
                                             kw.get("gi"), kw.get("bits", 3), kw.get("gs", 128),
                                             kw.get("v2", 0), kw.get("N", 5120), kw.get("K", 13824),
                                             kw.get("out", OUT))
    assert ok() == 0
    assert ok(out=None) == -1
    assert ok(bits=1) == -2
    assert ok(N=5121) == -3
    assert ok(gs=100) == -4
    assert ok(out=OUT + 8) == -5


@needs_lib
def test_convert_zeros_check_codes():
    lib = gq.library()
    ck = lambda i=QZ, o=OUT, b=4, G=8, N=4096, v=1, c=None: lib.gptq_convert_zeros_check(i, o, b, G, N, v, c)
    assert ck() == 0
    assert ck(o=QZ) == 0                          # in place
    assert ck(c=GI) == 0
    assert ck(i=None) == -1 and ck(o=None) == -1
    for b in (1, 5, 16):
        assert ck(b=b) == -2
    assert ck(G=0) == -3 and ck(N=0) == -3 and ck(N=48) == -3 and ck(N=1 << 21) == -3
    assert ck(v=2) == -9
    assert ck(o=QZ + 4) == -9                     # partial overlap
    assert ck(i=QZ + 2) == -5 and ck(c=GI + 2) == -5
    assert ck(b=3, N=32, G=1) == 0


def test_repack_argument_codes():
    """Bad repack arguments return before any launch (safe without a GPU)."""
    lib = gq.library()
    for fn in (lib.gptq_repack_tiled, lib.gptq_unrepack_tiled):
        assert fn(None, OUT, 4, 4096, 4096, None) == -1
        assert fn(QW, None, 4, 4096, 4096, None) == -1
        assert fn(QW, OUT, 5, 4096, 4096, None) == -2
        assert fn(QW, OUT, 4, 48, 4096, None) == -3
        assert fn(QW, OUT, 4, 4096, 4112, None) == -3
        assert fn(QW + 4, OUT, 4, 4096, 4096, None) == -5
        assert fn(QW, QW, 4, 4096, 4096, None) == -9          # in place
        assert fn(QW, QW + 16, 4, 64, 64, None) == -9         # overlap


def test_tiled_describe_shapes():
    """Tiled-layout plans: the M = 1 shapes picked from the layer sweeps, the
    general rules elsewhere, the prefill kernel for large M."""
    lib = gq.library()
    buf = ctypes.create_string_buffer(256)
    for (bits, gs, M, K, N, want) in ((4, 128, 1, 4096, 12288, "<4, false, 1, 1, 16, 4> grid=768 block=512"),
                                      (4, 128, 1, 4096, 22016, "<4, false, 1, 2, 16, 4> grid=688 block=512"),
                                      (4, 128, 1, 11008, 4096, "<4, false, 1, 1, 16, 4> grid=256 block=704 phases=2"),
                                      # K <= 2048: 4 waves of 16 chunks, no empty chunk slots
                                      (4, 128, 1, 2048, 4096, "<4, false, 1, 1, 16, 4> grid=256 block=256 phases=1"),
                                      (2, 64, 1, 2048, 16384, "<2, false, 1, 2, 16, 2> grid=512 block=256 phases=1"),
                                      (4, 128, 1, 3072, 4096, "<4, false, 1, 1, 16, 4> grid=256 block=512 phases=1"),
                                      (2, 64, 16, 4096, 12288, "<2, false, 4, "),
                                      (3, 128, 16, 5120, 13824, "<3, false, 4, ")):
        assert lib.gptq_gemm_tiled_describe(X, QW, QZ, SC, None, bits, gs, 1, M, N, K, OUT, 0, 0, buf, 256) == 0
        assert buf.value.decode().startswith("gptq::decode_kernel" + want), buf.value
    # 2048 x 8192: 8 x 32 tiles of 256 rows fit one round on 256 CUs (the 256-row tile,
    # 8-bit with its pipelined body); 2048 x 28672 needs several rounds (the 128-row tile,
    # 8-bit with the plain body)
    for (bits, N, want) in ((4, 8192, "gptq::prefill_big_kernel<4, true, true> grid=32x8"),
                            (4, 28672, "gptq::prefill_kernel<4, false, true, true> grid=112x16"),
                            (8, 8192, "gptq::prefill_big_kernel<8, true, false> grid=32x8"),
                            (8, 28672, "gptq::prefill_kernel<8, false, false, false> grid=112x16")):
        assert lib.gptq_gemm_tiled_describe(X, QW, QZ, SC, None, bits, 128, 1, 2048, N, 8192, OUT, 0, 0, buf, 256) == 0
        assert buf.value.decode().startswith(want), buf.value


def test_row_block_plans():
    """Host-only plan boundaries of the decode kernel over 16-row blocks:
    per-element layers (act order, or groups that are not whole 64-row k
    tiles) at 17..4096 rows; small fp16 fast-path layers (N, K bounded, at
    most 128 decode column tiles) at 17..64 rows; a forced prefill path and
    everything else keep the prefill kernel."""
    lib = gq.library()
    buf = ctypes.create_string_buffer(256)

    def plan(bits, gs, M, K, N, gi=None, tiled=True, path=0, bf16=False):
        if bf16:
            fn = lib.gptq_gemm_tiled_bf16_describe if tiled else lib.gptq_gemm_bf16_describe
        else:
            fn = lib.gptq_gemm_tiled_describe if tiled else lib.gptq_gemm_describe
        assert fn(X, QW, QZ, SC, gi, bits, gs, 1, M, N, K, OUT, path, 0, buf, 256) == 0
        return buf.value.decode()

    # per-element layers
    assert plan(4, 128, 17, 4096, 12288, GI).startswith("gptq::decode_kernel<4, true,")
    assert plan(4, 128, 17, 4096, 12288, GI).endswith("row_blocks=2")
    assert plan(3, 128, 4096, 5120, 13824, GI, tiled=False).endswith("row_blocks=256")
    assert plan(4, 128, 4097, 4096, 12288, GI).startswith("gptq::prefill_kernel<4, true,")
    assert plan(4, 32, 40, 4096, 12288).startswith("gptq::decode_kernel<4, false,")
    assert plan(4, 32, 40, 4096, 12288).endswith("row_blocks=3")
    assert plan(4, 128, 40, 4096, 1024, GI, bf16=True).startswith("gptq::decode_bf16_kernel")
    assert plan(4, 128, 17, 4096, 12288, GI, path=2).startswith("gptq::prefill_small_kernel<4, true,")
    # small fp16 fast-path layers
    assert plan(4, 128, 17, 4096, 4096).endswith("row_blocks=2")
    assert plan(4, 128, 64, 4096, 4096).endswith("row_blocks=4")
    assert plan(4, 128, 64, 8192, 1024).endswith("row_blocks=4")
    assert plan(4, 128, 65, 4096, 4096).startswith("gptq::prefill")           # rows past 64
    assert plan(4, 128, 17, 4096, 4096, tiled=False).startswith("gptq::prefill")   # 256 decode tiles
    assert plan(4, 128, 17, 11008, 4096).startswith("gptq::prefill")          # K past 8192
    assert plan(4, 128, 17, 4096, 8192).startswith("gptq::prefill")           # N past 4096
    assert plan(4, 128, 17, 4096, 12288).startswith("gptq::prefill")
    assert plan(4, 128, 17, 4096, 4096, bf16=True).startswith("gptq::prefill_bf16")
    assert plan(4, 128, 17, 4096, 4096, path=2).startswith("gptq::prefill_small_kernel")


def test_moe_argument_codes():
    """Bad grouped-GEMM arguments return before any launch (safe without a GPU)."""
    lib = gq.library()
    OFF = 0x70000
    mo = lambda x=X, qw=QW, qz=QZ, sc=SC, gi=None, off=OFF, E=8, mt=16, b=4, gs=128, v2=1, T=32, N=4096, K=4096, o=OUT: \
        lib.gptq_moe_gemm(x, qw, qz, sc, gi, off, E, mt, b, gs, v2, T, N, K, o, None)
    assert mo(off=None) == -1
    assert mo(qw=None) == -1
    assert mo(b=5) == -2
    assert mo(N=48) == -3
    assert mo(T=-1) == -3
    assert mo(gs=100) == -4
    assert mo(E=0) == -9
    assert mo(mt=-1) == -9
    assert mo(x=X + 8) == -5
    assert mo(off=OFF + 2) == -5
    assert mo(T=0, x=None, o=None) == 0               # nothing to do, nothing launched
    assert mo(mt=0) == 0
    mx = lambda path, **kw: lib.gptq_moe_gemm_ex(X, QW, QZ, SC, None, kw.get("off", OFF), 8, kw.get("mt", 16), 4, 128,
                                                  1, 32, 4096, 4096, OUT, None, path)
    assert mx(-1) == -9 and mx(3) == -9               # path out of range
    assert mx(1, off=None) == -1 and mx(2, off=None) == -1
    assert mx(2, mt=0) == 0 and mx(1, mt=0) == 0


def test_sorted_argument_codes():
    """Bad act-order sort / sorted GEMM arguments return before touching the device."""
    lib = gq.library()
    PERM = 0x80000
    assert lib.gptq_sort_act_order(QW, None, 4, 128, 4096, 4096, OUT, PERM, None) == -1
    assert lib.gptq_sort_act_order(QW, GI, 5, 128, 4096, 4096, OUT, PERM, None) == -2
    assert lib.gptq_sort_act_order(QW, GI, 4, 100, 4096, 4096, OUT, PERM, None) == -4
    assert lib.gptq_sort_act_order(QW, GI, 4, 128, 4096, 4096, OUT + 4, PERM, None) == -5
    assert lib.gptq_sort_act_order(QW, GI, 4, 128, 4096, 4096, QW, PERM, None) == -9     # in place
    sg = lambda perm=PERM, layout=0, path=0, K=4096: lib.gptq_gemm_sorted(X, QW, QZ, SC, perm, 4, 128, 1, 1, 4096, K,
                                                                          OUT, None, layout, path, 0)
    assert sg(perm=None) == -1
    assert sg(perm=PERM + 2) == -5
    assert sg(layout=2) == -9
    assert sg(path=3) == -9


def test_invalid_calls_return_before_any_launch():
    """gptq_gemm / gptq_dequant with bad arguments fail in the host checks, so
    they are safe to call without a GPU."""
    lib = gq.library()
    assert lib.gptq_gemm(X, QW, QZ, SC, None, 5, 128, 1, 1, 4096, 4096, OUT, None) == -2
    assert lib.gptq_gemm_ex(X, QW, QZ, SC, None, 4, 128, 1, 17, 4096, 4096, OUT, None, 1, 0) == -9
    assert lib.gptq_gemm_ex(X, QW, QZ, SC, None, 4, 128, 1, 1, 4096, 4096, OUT, None, 3, 0) == -9
    assert lib.gptq_gemm_ex(X, QW, QZ, SC, None, 4, 128, 1, 1, 4096, 4096, OUT, None, 0, -1) == -9
    assert lib.gptq_gemm_ex(X, QW, QZ, SC, None, 4, 128, 1, 1, 4096, 4096, OUT, None, 0, 17) == -9
    assert lib.gptq_dequant(QW, QZ, SC, None, 4, 100, 1, 4096, 4096, OUT, None) == -4
    assert lib.gptq_gemm(X, QW, QZ, SC, None, 4, 128, 1, 0, 4096, 4096, OUT, None) == 0   # M == 0


def test_python_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    qw = torch.zeros((512, 64), dtype=torch.int32)
    qz = torch.zeros((32, 8), dtype=torch.int32)
    sc = torch.zeros((32, 64), dtype=torch.float16)
    x = torch.zeros((1, 4096), dtype=torch.float16)
    with pytest.raises(ValueError):
        gq.gemm(x, qw, qz, sc, None, 5, 128, True)
    with pytest.raises(ValueError):
        gq.gemm(x, qw, qz, sc, None, 4, 128, True)          # CPU tensors are rejected


@needs_lib
def test_every_decode_shape_has_a_launch_plan():
    """Kernel choice and launch shape (pure host) succeed for every bit width,
    M in 1..16, both scale paths and the layer shapes the workloads use, plus
    ragged small ones."""
    shapes = [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096), (12288, 4096), (5120, 13824),
              (13824, 5120), (8192, 28672), (28672, 8192), (96, 32), (256, 160), (1024, 32), (32768, 64)]
    for bits in (2, 3, 4, 8):
        for K, N in shapes:
            for gi in (None, GI):
                for gs in (32, 128):
                    if K % gs:
                        continue
                    for M in list(range(1, 17)) + [17, 2048]:
                        rc = gemm_check(gi=gi, bits=bits, gs=gs, M=M, N=N, K=K)
                        assert rc == 0, (bits, K, N, gi, gs, M, rc)


@needs_lib
def test_forced_decode_always_has_a_launch_plan():
    """path = decode must find a launch shape for every M <= 16 and every waves
    setting, on the shapes the GPU tests force it on."""
    lib = gq.library()
    shapes = [(512, 160, 32), (512, 160, 128), (96, 32, 32), (96, 96, 96), (288, 224, 96), (256, 64, 16),
              (544, 96, 32), (1024, 32, 1024), (2048, 320, 128), (8192, 256, 128), (8192, 4608, 128),
              (8192, 17408, 128), (4096, 12288, 64), (12288, 4096, 64), (5120, 13824, 128), (13824, 5120, 128)]
    for bits in (2, 3, 4, 8):
        for K, N, gs in shapes:
            for gi in (None, GI):
                for M in range(1, 17):
                    for waves in (0, 1, 2, 3, 4, 8, 16):
                        rc = lib.gptq_gemm_ex_check(X, QW, QZ, SC, gi, bits, gs, 1, M, N, K, OUT, 1, waves)
                        assert rc == 0, (bits, K, N, gs, gi, M, waves, rc)


@needs_lib
def test_describe_names_the_kernel():
    lib = gq.library()
    buf = ctypes.create_string_buffer(256)
    assert lib.gptq_gemm_describe(X, QW, QZ, SC, None, 4, 128, 0, 1, 12288, 4096, OUT, 0, 0, buf, 256) == 0
    assert buf.value.decode().startswith("gptq::decode_kernel<4, false, 1, ")
    assert lib.gptq_gemm_describe(X, QW, QZ, SC, GI, 3, 128, 1, 16, 5120, 13824, OUT, 0, 0, buf, 256) == 0
    assert buf.value.decode().startswith("gptq::decode_kernel<3, true, 4, ")
    assert lib.gptq_gemm_describe(X, QW, QZ, SC, None, 8, 128, 1, 2048, 28672, 8192, OUT, 0, 0, buf, 256) == 0
    assert buf.value.decode().startswith("gptq::prefill_kernel<8, false, false, false>")
    assert lib.gptq_gemm_describe(X, QW, QZ, SC, None, 5, 128, 1, 1, 4096, 4096, OUT, 0, 0, buf, 256) == -2
    assert lib.gptq_gemm_describe(X, QW, QZ, SC, None, 4, 128, 1, 1, 4096, 4096, OUT, 0, 0, None, 256) == -1
    small = ctypes.create_string_buffer(8)
    assert lib.gptq_gemm_describe(X, QW, QZ, SC, None, 4, 128, 1, 1, 4096, 4096, OUT, 0, 0, small, 8) == 0
    assert len(small.value) == 7


@needs_lib
def test_describe_bf16_kernels():
    """bfloat16 activations: decode always on the element-wise bf16 kernel (no
    64-column tiles at one row), prefill on the bf16 twin of the fp16 tiles;
    the same argument checks."""
    lib = gq.library()
    buf = ctypes.create_string_buffer(256)
    for K, N in ((4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)):
        assert lib.gptq_gemm_bf16_describe(X, QW, QZ, SC, None, 4, 128, 0, 1, N, K, OUT, 0, 0, buf, 256) == 0
        d = buf.value.decode()
        assert d.startswith("gptq::decode_bf16_kernel<4, 1, ") and not d.startswith("gptq::decode_bf16_kernel<4, 1, 4,")
    assert lib.gptq_gemm_bf16_describe(X, QW, QZ, SC, GI, 3, 128, 1, 16, 5120, 13824, OUT, 0, 0, buf, 256) == 0
    assert buf.value.decode().startswith("gptq::decode_bf16_kernel<3, 4, ")
    assert lib.gptq_gemm_bf16_describe(X, QW, QZ, SC, None, 4, 128, 0, 2048, 28672, 8192, OUT, 0, 0, buf, 256) == 0
    assert buf.value.decode().startswith("gptq::prefill_bf16_kernel<4, false, true>")
    assert lib.gptq_gemm_bf16_describe(X, QW, QZ, SC, None, 5, 128, 1, 1, 4096, 4096, OUT, 0, 0, buf, 256) == -2
    assert lib.gptq_gemm_bf16_describe(X, QW, QZ, SC, None, 4, 100, 1, 1, 4096, 4096, OUT, 0, 0, buf, 256) == -4
    assert lib.gptq_dequant_bf16(QW, QZ, SC, None, 4, 100, 1, 4096, 4096, OUT, None) == -4
    assert lib.gptq_gemm_bf16(X, QW, QZ, SC, None, 4, 100, 1, 1, 4096, 4096, OUT, None) == -4
