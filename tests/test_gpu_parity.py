"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

- gptq_dequant must match the oracle bit for bit (compared as uint16);
- gptq_gemm must satisfy max|y - y_ref| <= 5e-3 * rms(y_ref), y_ref in fp64
  (tolerance of the GEMM target; fp32 accumulation on the GPU).

Inputs are seeded draws from ``workload`` quantized and packed by the oracle;
nothing the GPU computes is ever fed back to the oracle.
"""
import itertools

import numpy as np
import pytest

import oracle
import weight_only_bit_gptq_amd as gq
from workload import WORKLOADS, draw_layer, draw_workload_layer, random_words

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 8)
TOL = 5e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.library()
    return torch.device("cuda:0")


def k_splits(desc):
    """Split count a describe() string reports."""
    return int(desc.split("k_splits=")[1].split()[0])


def upload(L, dev):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return (t(L.qweight), t(L.qzeros), t(L.scales), None if L.g_idx is None else t(L.g_idx))


def quantized(K, N, M, bits, gs, sym, is_v2, act, seed=0, outliers=0.0, sigma=0.02):
    d = draw_layer(K, N, M, sigma=sigma, group_size=gs, outlier_rate=outliers, act_order=act, seed=seed)
    L = oracle.quantize_layer(d.W, bits, gs, sym, is_v2, d.g_idx)
    return d, L


def assert_close(y_gpu, y_ref, what=""):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all(), what
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.max(np.abs(y - y_ref))
    assert err <= TOL * rms, f"{what}: max err {err:.3e} > {TOL} * rms {rms:.3e}"


# ------------------------------------------------------------------ dequant, bit-exact
DQ_GRID = list(itertools.product(BITS, (False, True), (False, True), (False, True), (32, 64, 128)))


@pytest.mark.parametrize("bits,is_v2,sym,act,gs", DQ_GRID)
def test_dequant_bit_exact(dev, bits, is_v2, sym, act, gs):
    K, N = 256, 160                     # 2.5 column tiles, 8 chunks
    d, L = quantized(K, N, 1, bits, gs, sym, is_v2, act, seed=bits + 7 * gs)
    qw, qz, sc, gi = upload(L, dev)
    w = gq.dequant(qw, qz, sc, gi, bits, gs, is_v2)
    torch.cuda.synchronize()
    ref = oracle.dequant_ref(L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, is_v2, K, N)
    assert np.array_equal(w.cpu().numpy().view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("bits,is_v2", list(itertools.product(BITS, (False, True))))
def test_dequant_random_words_and_subnormals(dev, bits, is_v2):
    """Every field value (incl. top bits set, v1 zero 2^b - 1 -> 2^b) and scales
    whose products are fp16 subnormals."""
    K, N, gs = 192, 96, 64
    rng = np.random.default_rng(bits * 3 + is_v2)
    qweight = random_words(rng, (K * bits // 32, N))
    qzeros = random_words(rng, (K // gs, N * bits // 32))
    scales = (rng.standard_normal((K // gs, N)) * 0.05).astype(np.float16)
    scales[0, :32] = np.float16(2.0 ** -24) * np.arange(1, 33).astype(np.float16)
    scales[1, :8] = np.float16(-6.0e-8)
    t = lambda a: torch.from_numpy(a).to(dev)
    w = gq.dequant(t(qweight), t(qzeros), t(scales), None, bits, gs, is_v2)
    ref = oracle.dequant_ref(qweight, qzeros, scales, None, bits, gs, is_v2, K, N)
    assert np.array_equal(w.cpu().numpy().view(np.uint16), ref.view(np.uint16))


def test_dequant_v2_data_read_as_v1(dev):
    """Reading GPTQv2 zeros with is_v2 = 0 gives exactly the oracle's v1 reading
    (the misread of the v2 format is reproducible, never silent noise)."""
    bits, K, N, gs = 2, 256, 64, 64
    d, L = quantized(K, N, 1, bits, gs, False, True, False, seed=4, outliers=0.02)
    qw, qz, sc, gi = upload(L, dev)
    w = gq.dequant(qw, qz, sc, gi, bits, gs, False)
    ref_v1 = oracle.dequant_ref(L.qweight, L.qzeros, L.scales, None, bits, gs, False, K, N)
    ref_v2 = oracle.dequant_ref(L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N)
    assert np.array_equal(w.cpu().numpy().view(np.uint16), ref_v1.view(np.uint16))
    assert not np.array_equal(ref_v1.view(np.uint16), ref_v2.view(np.uint16))


# ------------------------------------------------------------------ GEMM, small grid
GEMM_GRID = list(itertools.product(BITS, (False, True), (False, True), (32, 128)))


@pytest.mark.parametrize("bits,is_v2,act,gs", GEMM_GRID)
def test_gemm_small_grid(dev, bits, is_v2, act, gs):
    K, N = 512, 160
    for sym in (False, True):
        d, L = quantized(K, N, 40, bits, gs, sym, is_v2, act, seed=bits * 11 + gs)
        qw, qz, sc, gi = upload(L, dev)
        xt = torch.from_numpy(d.x).to(dev)
        for M in (1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 40):
            ref = oracle.gptq_gemm_ref(d.x[:M], L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, is_v2, K, N)
            paths = [gq.PATH_AUTO, gq.PATH_PREFILL] + ([gq.PATH_DECODE] if M <= 16 else [])
            for p in paths:
                y = gq.gemm(xt[:M].contiguous(), qw, qz, sc, gi, bits, gs, is_v2, path=p)
                assert_close(y, ref, f"M={M} path={p} sym={sym}")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,N,gs", [(96, 32, 32), (96, 96, 96), (288, 224, 96), (256, 64, 16), (544, 96, 32),
                                    (1024, 32, 1024)])
def test_gemm_ragged_and_group_shapes(dev, bits, K, N, gs):
    """Ragged K (not a multiple of the 128-row wave step or the 64-row prefill
    tile), N with a half column tile, and group sizes 16 / 96 / K that are not
    multiples of the 32- and 64-row pipelines (per-element path)."""
    d, L = quantized(K, N, 33, bits, gs, False, True, False, seed=K + N + gs)
    qw, qz, sc, gi = upload(L, dev)
    xt = torch.from_numpy(d.x).to(dev)
    for M in (1, 7, 16, 33):
        ref = oracle.gptq_gemm_ref(d.x[:M], L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N)
        for p in ([gq.PATH_DECODE] if M <= 16 else []) + [gq.PATH_PREFILL]:
            y = gq.gemm(xt[:M].contiguous(), qw, qz, sc, gi, bits, gs, True, path=p)
            assert_close(y, ref, f"M={M} path={p}")


@pytest.mark.parametrize("waves", [1, 2, 3, 4, 8, 16])
def test_decode_waves_and_determinism(dev, waves):
    """Every waves-per-workgroup split of K gives the oracle's result, and
    repeated calls are bit-identical (fixed reduction order)."""
    bits, K, N, gs = 4, 2048, 320, 128
    d, L = quantized(K, N, 16, bits, gs, True, False, False, seed=21)
    qw, qz, sc, gi = upload(L, dev)
    xt = torch.from_numpy(d.x).to(dev)
    for M in (1, 2, 3, 4, 16):
        ref = oracle.gptq_gemm_ref(d.x[:M], L.qweight, L.qzeros, L.scales, None, bits, gs, False, K, N)
        x = xt[:M].contiguous()
        y1 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False, path=gq.PATH_DECODE, decode_waves=waves)
        y2 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False, path=gq.PATH_DECODE, decode_waves=waves)
        assert_close(y1, ref, f"M={M} waves={waves}")
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_multi_phase_k(dev, bits, M):
    """K long enough that M * K x-rows are staged in several LDS phases, with
    column tile widths of 16, 32 and 64 (N chosen to select each)."""
    K, gs = 8192, 128
    for N in (256, 4096 + 512, 16384 + 1024):
        if N > 5000 and bits != 4:
            continue
        d, L = quantized(K, N, M, bits, gs, False, True, False, seed=N + bits)
        qw, qz, sc, gi = upload(L, dev)
        cols = np.arange(0, N, max(1, N // 96))
        ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N, cols=cols)
        y = gq.gemm(torch.from_numpy(d.x).to(dev), qw, qz, sc, gi, bits, gs, True, path=gq.PATH_DECODE)
        assert_close(y[:, torch.from_numpy(cols).to(dev)], ref, f"N={N}")


FOLD_CASES = [
    # bits, gs, M, K, N, waves, tiled: group rows spanning 2 blocks (gs 256), blocks of 2 (gs 64),
    # no block fold (gs 96, 32), K splits whose length is not a multiple of 4 chunks, several rows
    (4, 256, 1, 2048, 256, 0, False), (4, 64, 1, 1024, 256, 0, True), (4, 96, 1, 960, 128, 0, False),
    (3, 32, 1, 512, 96, 0, False), (4, 128, 1, 11008, 1024, 0, False), (2, 128, 1, 12288, 512, 0, True),
    (3, 256, 4, 4096, 224, 0, False), (2, 64, 16, 4096, 256, 0, True), (8, 128, 7, 2048, 160, 3, False),
    (4, 128, 16, 11008, 1536, 0, True), (4, 256, 2, 8192, 96, 5, False),
    # K splits starting in the middle of a group (36 and 70 chunks per split, 8 chunks per group)
    (4, 256, 1, 9216, 256, 0, False), (4, 256, 1, 13312, 512, 0, False)]


@pytest.mark.parametrize("bits,gs,M,K,N,waves,tiled", FOLD_CASES)
def test_decode_block_fold(dev, bits, gs, M, K, N, waves, tiled):
    """Decode fast path with the scale and zero folded once per block of 2 or
    4 chunks: the fold the launch uses (the last template argument) divides
    the chunks per group and is 1 where the group is not a multiple of 64
    rows; oracle parity (asymmetric GPTQv1 data, zeros up to 2^b) on every
    column, repeated calls bit-identical."""
    d, L = quantized(K, N, M, bits, gs, False, False, False, seed=K + 3 * N + M)
    qw, qz, sc, gi = upload(L, dev)
    if tiled:
        qw = gq.repack_tiled(qw, bits)
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, False, path=gq.PATH_DECODE, decode_waves=waves)
    fold = int(desc.split(">")[0].split(",")[-1])
    cpg = gs // 32
    assert fold in (1, 2, 4) and cpg % fold == 0, desc
    if gs % 64 != 0:
        assert fold == 1, desc
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, False, K, N)
    y1 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False, path=gq.PATH_DECODE, decode_waves=waves)
    y2 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False, path=gq.PATH_DECODE, decode_waves=waves)
    assert_close(y1, ref, desc)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), desc


@pytest.mark.parametrize("bits,gs,K,N", [(4, 128, 2048, 4096), (2, 64, 2048, 8192), (3, 128, 2048, 2048),
                                         (8, 128, 1024, 2048), (4, 32, 1024, 16384)])
def test_decode_tiled_short_k_four_waves(dev, bits, gs, K, N):
    """Tiled layout, one row, K <= 2048: the planner takes 4 waves of 16
    chunks (no wave without chunks; 8 waves would leave half their slots
    empty); oracle parity on every column, repeated calls bit-identical."""
    d, L = quantized(K, N, 1, bits, gs, True, False, False, seed=K + N + bits)
    qw, qz, sc, gi = upload(L, dev)
    qw = gq.repack_tiled(qw, bits)
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, False)
    assert desc.startswith("gptq::decode_kernel") and " block=256 " in desc and "phases=1 " in desc, desc
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, False, K, N)
    y1 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)
    y2 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)
    assert_close(y1, ref, desc)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), desc


SPLIT_CASES = [(4, 128, 1, 8192, 512, False), (4, 128, 3, 8192, 96, False), (8, 128, 7, 8192, 512, True),
               (2, 64, 4, 12288, 1024, False), (3, 128, 16, 13824, 640, True), (4, 128, 1, 11008, 1024, False),
               (3, 32, 2, 9216, 352, False), (4, 128, 16, 8192, 1536, False)]


@pytest.mark.parametrize("bits,gs,M,K,N,act", SPLIT_CASES)
def test_decode_split_k(dev, bits, gs, M, K, N, act):
    """Shapes whose launch splits K over several workgroups per column tile:
    oracle parity on sampled columns, bit-identical repeated calls (fixed
    split order), and a second call that rewrites every output (the arrival
    counters are re-armed by the first)."""
    d, L = quantized(K, N, M, bits, gs, False, True, act, seed=K + N + M)
    qw, qz, sc, gi = upload(L, dev)
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_DECODE)
    assert k_splits(desc) > 1, desc
    cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 80)), [N - 1]]))
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N, cols=cols)
    y1 = gq.gemm(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_DECODE)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    y2 = gq.gemm(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_DECODE, out=out)
    assert_close(y1[:, torch.from_numpy(cols).to(dev)], ref, desc)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), desc


PREFILL_SPLIT_CASES = [
    # bits, gs, M, K, N, act, tiled: small-M prefill grids whose tiles split K
    # (fast path, per-element path through act order and 32-row groups, a K
    # with a last half k tile, two-word blocks, ragged rows and columns)
    (4, 128, 17, 4096, 1024, False, True), (4, 128, 64, 2048, 512, False, False),
    (3, 128, 33, 4096, 256, True, False), (8, 128, 20, 2048, 768, False, True),
    (2, 64, 50, 4096, 512, False, False), (4, 32, 40, 2048, 256, False, False),
    (4, 32, 24, 2080, 288, False, True), (3, 128, 130, 8192, 160, False, True),
    (4, 128, 17, 16384, 256, False, False),
    # the sum kernel's four widths: up to 4, 8, 16 and 32 splits (4 and 8 here;
    # 28 and 26, below 32, repeat the last split's loads without adding them)
    (4, 128, 100, 1024, 8192, False, False), (3, 128, 48, 2048, 6144, False, True),
    (4, 64, 24, 1024, 6144, False, True), (4, 128, 24, 7168, 512, False, True),
    (2, 128, 17, 6656, 512, False, False)]


@pytest.mark.parametrize("bits,gs,M,K,N,act,tiled", PREFILL_SPLIT_CASES)
def test_prefill_split_k(dev, bits, gs, M, K, N, act, tiled):
    """Prefill launches whose grid of output tiles is small split K over
    several workgroups per tile (a second kernel adds the fp32 partial sums in
    split order): oracle parity on every column, bit-identical repeated calls,
    a second call that rewrites every output, and the same result from a graph
    captured after the stream has its workspace, replayed three times."""
    d, L = quantized(K, N, M, bits, gs, False, True, act, seed=K + 7 * N + M)
    qw, qz, sc, gi = upload(L, dev)
    if tiled:
        qw = gq.repack_tiled(qw, bits)
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_PREFILL)
    assert desc.startswith(("gptq::prefill_kernel", "gptq::prefill_small_kernel")), desc
    assert k_splits(desc) > 1, desc
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N)
    y1 = gq.gemm(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_PREFILL)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    y2 = gq.gemm(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_PREFILL, out=out)
    assert_close(y1, ref, desc)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), desc
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gq.gemm(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_PREFILL)   # the stream's workspace
    s.synchronize()
    outg = torch.zeros((M, N), dtype=torch.float16, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gq.gemm(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_PREFILL, out=outg)
    for _ in range(3):
        outg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outg.view(torch.int16), y1.view(torch.int16)), desc


ROW_BLOCK_CASES = [
    # bits, gs, M, K, N, act, tiled: per-element layers above 16 rows run the
    # decode kernel over blocks of 16 rows (ragged last blocks; column tile
    # counts with and without whole eighths, i.e. both workgroup mappings;
    # act order, and 32- / 96-row groups on the fast path)
    (3, 128, 17, 2048, 256, True, False), (4, 128, 40, 1024, 288, True, True), (2, 64, 100, 1024, 512, True, False),
    (8, 128, 33, 1024, 256, True, True), (4, 32, 48, 2048, 1024, False, False), (4, 96, 70, 1152, 256, False, True),
    (3, 32, 256, 1024, 256, False, True), (4, 128, 20, 8192, 256, True, False)]


@pytest.mark.parametrize("bits,gs,M,K,N,act,tiled", ROW_BLOCK_CASES)
def test_decode_row_blocks(dev, bits, gs, M, K, N, act, tiled):
    """gptq_gemm's automatic plan for these layers is the decode kernel over
    ceil(M / 16) row blocks: oracle parity on every output, bit-identical
    repeats, and the same result through a graph replayed twice."""
    d, L = quantized(K, N, M, bits, gs, False, True, act, seed=K + N + M + gs)
    qw, qz, sc, gi = upload(L, dev)
    if tiled:
        qw = gq.repack_tiled(qw, bits)
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, True)
    assert desc.startswith("gptq::decode_kernel") and f"row_blocks={(M + 15) // 16}" in desc, desc
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N)
    y1 = gq.gemm(x, qw, qz, sc, gi, bits, gs, True)
    assert_close(y1, ref, desc)
    y2 = gq.gemm(x, qw, qz, sc, gi, bits, gs, True)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        gq.gemm(x, qw, qz, sc, gi, bits, gs, True, out=out)
    for _ in range(2):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("bits,gs,M,K,N,tiled,want", [
    (4, 128, 24, 1024, 1024, True, "row_blocks=2"), (2, 64, 32, 2048, 512, False, "row_blocks=2"),
    (8, 128, 17, 1024, 768, True, "row_blocks=2"), (4, 128, 17, 4096, 4096, True, "row_blocks=2"),
    (4, 128, 50, 2048, 1024, True, "row_blocks=4"), (3, 128, 64, 1024, 512, False, "row_blocks=4"),
    # excluded: more than 128 column tiles (checkpoint 4096 -> 4096), rows past 64, long K
    (4, 128, 17, 4096, 4096, False, "gptq::prefill"), (4, 128, 65, 1024, 1024, True, "gptq::prefill"),
    (4, 128, 17, 11008, 512, True, "gptq::prefill")])
def test_small_layer_row_blocks(dev, bits, gs, M, K, N, tiled, want):
    """Small fast-path layers at 17-64 rows take the decode kernel over row
    blocks when its plan has at most 128 column tiles, else the prefill
    kernel: the plan, and oracle parity on every output."""
    d, L = quantized(K, N, M, bits, gs, False, True, False, seed=K + N + M + bits)
    qw, qz, sc, gi = upload(L, dev)
    if tiled:
        qw = gq.repack_tiled(qw, bits)
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, True)
    assert want in desc and (not want.startswith("row_blocks") or desc.startswith("gptq::decode_kernel")), desc
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N)
    assert_close(gq.gemm(x, qw, qz, sc, gi, bits, gs, True), ref, desc)


def test_decode_row_blocks_full_size(dev):
    """Llama-7B qkv (4096 -> 12288, 4-bit g128) with act-order g_idx at 600
    rows, tiled: the decode kernel over 38 row blocks (the last of 8 rows);
    oracle parity on sampled columns, computed one by one."""
    K, N, M, bits, gs = 4096, 12288, 600, 4, 128
    d, L = quantized(K, N, M, bits, gs, True, False, True, seed=600)
    qw, qz, sc, gi = upload(L, dev)
    qw = gq.repack_tiled(qw, bits)
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, False)
    assert desc.startswith("gptq::decode_kernel<4, true,") and "row_blocks=38" in desc, desc
    cols = np.unique(np.concatenate([np.arange(0, N, 101), [N - 1]]))
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, False, K, N, cols=cols)
    y = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)
    assert_close(y[:, torch.from_numpy(cols).to(dev)], ref, desc)


def test_decode_row_blocks_bf16(dev):
    """bfloat16 act-order layer at 40 rows: the decode kernel over row blocks,
    within the bf16 bar (the element-wise bf16 dequant, fp32 sums)."""
    K, N, M, bits, gs = 1024, 256, 40, 4, 128
    d, L = quantized(K, N, M, bits, gs, False, True, True, seed=41)
    sc_b = torch.from_numpy(L.scales.astype(np.float32)).to(torch.bfloat16)
    x_b = torch.from_numpy(d.x.astype(np.float32)).to(torch.bfloat16)
    qw, qz, _, gi = upload(L, dev)
    desc = gq.describe(x_b.to(dev), qw, qz, sc_b.to(dev), gi, bits, gs, True)
    assert desc.startswith("gptq::decode_bf16_kernel") and "row_blocks=3" in desc, desc
    ref = oracle.gptq_gemm_ref(x_b.double().numpy(), L.qweight, L.qzeros, sc_b.double().numpy(), L.g_idx, bits, gs,
                               True, K, N, act="bf16")
    y = gq.gemm(x_b.to(dev), qw, qz, sc_b.to(dev), gi, bits, gs, True).to(torch.float64).cpu().numpy()
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(y - ref) <= TOL * rms + 2.0 ** -8 * np.abs(ref)), desc


def test_prefill_split_k_full_size_small_batch(dev):
    """Llama-7B qkv at 17 and 128 rows (tiled layout, the automatic plan: the
    32-row and the 128-row prefill tile, K split 8 and 5 ways): oracle parity
    on sampled columns, computed one by one."""
    wl = WORKLOADS["llama7b_decode_w4g128"]
    layer = wl.layers[0]
    d = draw_workload_layer(wl, layer, 128, seed=3)
    L = oracle.quantize_layer(d.W, wl.bits, wl.group_size, wl.sym, wl.is_v2, d.g_idx)
    qw, qz, sc, gi = upload(L, dev)
    qw = gq.repack_tiled(qw, wl.bits)
    cols = np.unique(np.concatenate([np.arange(0, layer.N, 97), [layer.N - 1]]))
    for M in (17, 128):
        x = torch.from_numpy(d.x[:M]).to(dev)
        desc = gq.describe(x, qw, qz, sc, gi, wl.bits, wl.group_size, wl.is_v2)
        assert k_splits(desc) > 1, desc
        ref = oracle.gptq_gemm_ref(d.x[:M], L.qweight, L.qzeros, L.scales, None, wl.bits, wl.group_size, wl.is_v2,
                                   layer.K, layer.N, cols=cols)
        y = gq.gemm(x, qw, qz, sc, gi, wl.bits, wl.group_size, wl.is_v2)
        assert_close(y[:, torch.from_numpy(cols).to(dev)], ref, desc)


def test_decode_split_k_alternating_shapes(dev):
    """Split-K calls of different shapes (different partial-sum sizes and tile
    counts) alternate on one stream and share its workspace; every call must
    find its tiles' arrival counters at zero and leave them so."""
    layers = []
    for (bits, gs, M, K, N) in ((4, 128, 1, 8192, 1024), (4, 128, 4, 8192, 96), (2, 64, 1, 8192, 1024)):
        d, L = quantized(K, N, M, bits, gs, False, True, False, seed=N + M)
        qw, qz, sc, gi = upload(L, dev)
        x = torch.from_numpy(d.x).to(dev)
        assert k_splits(gq.describe(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_DECODE)) > 1
        cols = np.arange(0, N, max(1, N // 64))
        ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N, cols=cols)
        layers.append((x, qw, qz, sc, bits, gs, M, N, cols, ref))
    for rep in range(3):
        for i in (2, 0, 1, 0, 2, 1):
            x, qw, qz, sc, bits, gs, M, N, cols, ref = layers[i]
            out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
            gq.gemm(x, qw, qz, sc, None, bits, gs, True, path=gq.PATH_DECODE, out=out)
            assert_close(out[:, torch.from_numpy(cols).to(dev)], ref, f"rep {rep} layer {i}")


def test_decode_split_k_other_stream_and_graph(dev):
    """A split-K call on a new stream (its own workspace) and inside a captured
    graph on a stream that never ran eagerly (no workspace yet: the call falls
    back to one split) both match the default-stream result."""
    bits, gs, M, K, N = 4, 128, 1, 8192, 512
    d, L = quantized(K, N, M, bits, gs, True, False, False, seed=77)
    qw, qz, sc, gi = upload(L, dev)
    x = torch.from_numpy(d.x).to(dev)
    y0 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)
    s.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    s2 = torch.cuda.Stream()
    out = torch.zeros((M, N), dtype=torch.float16, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s2):
        gq.gemm(x, qw, qz, sc, gi, bits, gs, False, out=out)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert_close(out, y0.float().cpu().numpy().astype(np.float64), "graph replay")



def test_workspace_growth_keeps_captured_graph(dev):
    """A graph captured on stream s keeps the workspace s had at capture time.
    A later eager call on s that needs a larger workspace (a sorted act-order
    call gathering a big x) replaces it, and the replaced buffer must stay
    allocated: replays after the growth still match the eager result bit for
    bit (same kernel, same split order) and the oracle."""
    bits, gs, M, K, N = 4, 128, 1, 8192, 512
    d, L = quantized(K, N, M, bits, gs, True, False, False, seed=78)
    qw, qz, sc, gi = upload(L, dev)
    x = torch.from_numpy(d.x).to(dev)
    assert k_splits(gq.describe(x, qw, qz, sc, gi, bits, gs, False)) > 1
    cols = np.arange(0, N, 7)
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, False, K, N, cols=cols)
    # a big act-order layer for the eager call that grows the workspace
    Kb, Nb, Mb = 4096, 64, 512
    db, Lb = quantized(Kb, Nb, Mb, bits, gs, False, True, True, seed=79)
    qwb, qzb, scb, gib = upload(Lb, dev)
    qsb, permb = gq.sort_act_order(qwb, gib, bits, gs)
    xb = torch.from_numpy(db.x).to(dev)
    colsb = np.arange(0, Nb, 5)
    refb = oracle.gptq_gemm_ref(db.x, Lb.qweight, Lb.qzeros, Lb.scales, Lb.g_idx, bits, gs, True, Kb, Nb, cols=colsb)
    s = torch.cuda.Stream()
    out = torch.zeros((M, N), dtype=torch.float16, device=dev)
    with torch.cuda.stream(s):
        y_eager = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)       # allocates s's workspace (split K)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gq.gemm(x, qw, qz, sc, gi, bits, gs, False, out=out)
    with torch.cuda.stream(s):
        yb = gq.gemm_sorted(xb, qsb, qzb, scb, permb, bits, gs, True)   # Mb * Kb * 2 = 4 MiB: grows it
    s.synchronize()
    assert_close(yb[:, torch.from_numpy(colsb).to(dev)], refb, "sorted call that grew the workspace")
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep}"
        assert_close(out[:, torch.from_numpy(cols).to(dev)], ref, f"replay {rep}")


def test_workspace_allocation_failure(dev, monkeypatch):
    """With workspace allocation failing (the library's GPTQ_TEST_FAIL_WORKSPACE
    hook), a split-K decode call on a stream without a workspace runs unsplit
    (documented fallback, same result within tolerance) and a sorted act-order
    call reports GPTQ_ERR_NO_MEM; once allocation works again both succeed."""
    bits, gs, M, K, N = 4, 128, 1, 8192, 512
    d, L = quantized(K, N, M, bits, gs, True, False, False, seed=80)
    qw, qz, sc, gi = upload(L, dev)
    x = torch.from_numpy(d.x).to(dev)
    assert k_splits(gq.describe(x, qw, qz, sc, gi, bits, gs, False)) > 1
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, False, K, N)
    da, La = quantized(1024, 64, 4, bits, gs, False, True, True, seed=81)
    qwa, qza, sca, gia = upload(La, dev)
    qsa, perma = gq.sort_act_order(qwa, gia, bits, gs)
    xa = torch.from_numpy(da.x).to(dev)
    refa = oracle.gptq_gemm_ref(da.x, La.qweight, La.qzeros, La.scales, La.g_idx, bits, gs, True, 1024, 64)
    s = torch.cuda.Stream()
    monkeypatch.setenv("GPTQ_TEST_FAIL_WORKSPACE", "1")
    with torch.cuda.stream(s):
        y = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)
        with pytest.raises(gq.GptqError) as err:
            gq.gemm_sorted(xa, qsa, qza, sca, perma, bits, gs, True)
    s.synchronize()
    assert err.value.code == -6
    assert_close(y, ref, "unsplit fallback")
    monkeypatch.delenv("GPTQ_TEST_FAIL_WORKSPACE")
    with torch.cuda.stream(s):
        y2 = gq.gemm(x, qw, qz, sc, gi, bits, gs, False)
        ya = gq.gemm_sorted(xa, qsa, qza, sca, perma, bits, gs, True)
    s.synchronize()
    assert_close(y2, ref, "split after the hook is off")
    assert_close(ya, refa, "sorted after the hook is off")

# ------------------------------------------------------------------ tiled qweight layout
@pytest.mark.parametrize("bits", BITS)
def test_repack_tiled_bit_exact(dev, bits):
    """gptq_repack_tiled reproduces the oracle's tiled layout exactly (words
    moved, 4-bit fields in pair order) and gptq_unrepack_tiled inverts it."""
    for K, N in ((96, 32), (4096, 544), (11008, 64)):
        qw = random_words(np.random.default_rng(K + N + bits), (K * bits // 32, N))
        t = torch.from_numpy(qw).to(dev)
        tiled = gq.repack_tiled(t, bits)
        assert np.array_equal(tiled.cpu().numpy(), oracle.repack_tiled(qw, bits)), (K, N)
        assert torch.equal(gq.unrepack_tiled(tiled, bits), t), (K, N)


def upload_tiled(L, dev):
    """The layer with qweight in the tiled layout, permuted by the oracle."""
    qw, qz, sc, gi = upload(L, dev)
    return torch.from_numpy(oracle.repack_tiled(L.qweight, L.bits)).to(dev), qz, sc, gi


@pytest.mark.parametrize("bits,act,gs", list(itertools.product(BITS, (False, True), (32, 128))))
def test_gemm_tiled_small_grid(dev, bits, act, gs):
    """GEMM on the tiled layout: oracle parity on every path; the prefill
    result equals the checkpoint layout's bit for bit (same kernel, same
    order, only the weight addresses differ)."""
    K, N = 512, 160
    d, L = quantized(K, N, 40, bits, gs, False, True, act, seed=bits * 7 + gs)
    qw, qz, sc, gi = upload(L, dev)
    qt = upload_tiled(L, dev)[0]
    xt = torch.from_numpy(d.x).to(dev)
    for M in (1, 3, 16, 17, 40):
        ref = oracle.gptq_gemm_ref(d.x[:M], L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N)
        x = xt[:M].contiguous()
        for p in [gq.PATH_AUTO, gq.PATH_PREFILL] + ([gq.PATH_DECODE] if M <= 16 else []):
            y = gq.gemm(x, qt, qz, sc, gi, bits, gs, True, path=p)
            assert_close(y, ref, f"tiled M={M} path={p}")
        yt = gq.gemm(x, qt, qz, sc, gi, bits, gs, True, path=gq.PATH_PREFILL)
        yc = gq.gemm(x, qw, qz, sc, gi, bits, gs, True, path=gq.PATH_PREFILL)
        assert torch.equal(yt.view(torch.int16), yc.view(torch.int16)), f"M={M}"


@pytest.mark.parametrize("bits,gs,M,K,N,act", [(4, 32, 7, 96, 32, False), (3, 96, 5, 288, 224, False),
                                               (2, 16, 2, 256, 64, False), (4, 128, 1, 8192, 512, False),
                                               (8, 128, 7, 11008, 1024, True), (4, 128, 1, 4096, 4096, False),
                                               (2, 64, 16, 4096, 2048, False), (3, 128, 16, 5120, 1024, True)])
def test_gemm_tiled_shapes(dev, bits, gs, M, K, N, act):
    """Tiled layout at ragged, per-element, split-K and full-width shapes
    (sampled columns against the oracle)."""
    d, L = quantized(K, N, M, bits, gs, False, True, act, seed=K + N + gs)
    qt, qz, sc, gi = upload_tiled(L, dev)
    x = torch.from_numpy(d.x).to(dev)
    cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 96)), [N - 1]]))
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N, cols=cols)
    desc = gq.describe(x, qt, qz, sc, gi, bits, gs, True, path=gq.PATH_DECODE)
    y = gq.gemm(x, qt, qz, sc, gi, bits, gs, True, path=gq.PATH_DECODE)
    assert_close(y[:, torch.from_numpy(cols).to(dev)], ref, desc)



@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M,K,N", [(1024, 512, 12288), (1057, 576, 12320), (2048, 1024, 6144)])
def test_prefill_big_tiles(dev, bits, M, K, N):
    """Large M whose 256-row tiles fill one round of 3/4 .. all of the CUs
    takes the 256-row prefill tile (8-bit with its pipelined body, which only
    this tile holds without spills): ragged rows (M % 256) and columns
    (N % 256), both qweight layouts, against the oracle on sampled columns;
    the two layouts give the same bits."""
    gs = 64
    d, L = quantized(K, N, M, bits, gs, False, True, False, seed=M + K + N + bits)
    qw, qz, sc, gi = upload(L, dev)
    qt = upload_tiled(L, dev)[0]
    x = torch.from_numpy(d.x).to(dev)
    desc = gq.describe(x, qw, qz, sc, gi, bits, gs, True)
    assert desc.startswith(f"gptq::prefill_big_kernel<{bits}, true,"), desc
    cols = np.unique(np.concatenate([np.arange(0, N, 7), [N - 1]]))
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N, cols=cols)
    yc = gq.gemm(x, qw, qz, sc, gi, bits, gs, True)
    yt = gq.gemm(x, qt, qz, sc, gi, bits, gs, True)
    assert_close(yc[:, torch.from_numpy(cols).to(dev)], ref, desc)
    assert torch.equal(yc.view(torch.int16), yt.view(torch.int16)), desc

# ------------------------------------------------------------------ act-order rows sorted by group
@pytest.mark.parametrize("bits", BITS)
def test_sort_act_order_bit_exact(dev, bits):
    """gptq_sort_act_order reproduces the oracle's perm and sorted packed rows."""
    K, N, gs = 512, 96, 128
    d, L = quantized(K, N, 1, bits, gs, False, True, True, seed=bits + 70)
    qw, qz, sc, gi = upload(L, dev)
    want_q, want_p = oracle.sort_act_order(L.qweight, L.g_idx, bits, gs, K)
    qs, perm = gq.sort_act_order(qw, gi, bits, gs)
    assert np.array_equal(perm.cpu().numpy(), want_p)
    assert np.array_equal(qs.cpu().numpy(), want_q)


def test_sort_act_order_rejects_unequal_groups(dev):
    K, N, gs, bits = 256, 64, 64, 4
    d, L = quantized(K, N, 1, bits, gs, False, True, True, seed=3)
    qw, qz, sc, gi = upload(L, dev)
    bad = gi.clone()
    bad[0] = (int(bad[0]) + 1) % (K // gs)
    with pytest.raises(gq.GptqError):
        gq.sort_act_order(qw, bad, bits, gs)


@pytest.mark.parametrize("bits,M,tiled", [(3, 16, False), (3, 16, True), (4, 1, False), (4, 1, True),
                                          (2, 5, False), (8, 16, True), (4, 40, False), (3, 33, True)])
def test_gemm_sorted_matches_act_order(dev, bits, M, tiled):
    """The sorted act-order layer with x gathered by perm gives the act-order
    GEMM of the original layer (oracle), on the decode and prefill paths."""
    K, N, gs = 1024, 160, 128
    d, L = quantized(K, N, M, bits, gs, False, True, True, seed=bits * 3 + M)
    qw, qz, sc, gi = upload(L, dev)
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N)
    qs, perm = gq.sort_act_order(qw, gi, bits, gs)
    if tiled:
        qs = gq.repack_tiled(qs, bits)
    x = torch.from_numpy(d.x).to(dev)
    for p in [gq.PATH_AUTO, gq.PATH_PREFILL] + ([gq.PATH_DECODE] if M <= 16 else []):
        y = gq.gemm_sorted(x, qs, qz, sc, perm, bits, gs, True, path=p)
        assert_close(y, ref, f"path={p}")


def test_gemm_sorted_full_size_actorder(dev):
    """3-bit act-order decode layers at full size (5120 -> 13824 and
    13824 -> 5120, M = 16), sorted and tiled: sampled columns."""
    from workload import WORKLOADS
    wl = WORKLOADS["actorder_decode_w3g128"]
    for layer in wl.layers:
        d = draw_workload_layer(wl, layer, 16, seed=0)
        L = oracle.quantize_layer(d.W, wl.bits, wl.group_size, wl.sym, wl.is_v2, d.g_idx)
        qw, qz, sc, gi = upload(L, dev)
        qs, perm = gq.sort_act_order(qw, gi, wl.bits, wl.group_size)
        qs = gq.repack_tiled(qs, wl.bits)
        cols = np.arange(0, layer.N, 97)
        ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, wl.bits, wl.group_size, wl.is_v2,
                                   layer.K, layer.N, cols=cols)
        y = gq.gemm_sorted(torch.from_numpy(d.x).to(dev), qs, qz, sc, perm, wl.bits, wl.group_size, wl.is_v2)
        assert_close(y[:, torch.from_numpy(cols).to(dev)], ref, layer.name)


# ------------------------------------------------------------------ grouped (MoE) decode
def moe_problem(E, K, N, counts, bits, gs, act, seed, sym=False, is_v2=True):
    """E experts quantized by the oracle; tokens sorted by expert, `counts[e]` rows each."""
    experts = []
    for e in range(E):
        d = draw_layer(K, N, 1, sigma=0.02, group_size=gs, act_order=act, seed=seed + e)
        experts.append(oracle.quantize_layer(d.W, bits, gs, sym, is_v2, d.g_idx))
    T = int(sum(counts))
    x = draw_layer(K, N, max(T, 1), sigma=0.02, group_size=gs, seed=seed + 1000).x[:T]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return experts, x, offsets


def moe_upload(experts, x, offsets, act, dev):
    st = lambda name: torch.from_numpy(np.ascontiguousarray(np.stack([getattr(L, name) for L in experts]))).to(dev)
    gi = st("g_idx") if act else None
    return (torch.from_numpy(x).to(dev), st("qweight"), st("qzeros"), st("scales"), gi,
            torch.from_numpy(offsets).to(dev))


@pytest.mark.parametrize("bits,gs,act", [(4, 128, False), (4, 32, False), (2, 64, False), (3, 128, True),
                                         (8, 128, False), (4, 96, False)])
def test_moe_gemm_parity(dev, bits, gs, act):
    """Routed rows match the oracle expert by expert; experts with no rows,
    with more than 16 rows (several blocks) and rows after the last expert."""
    E, K, N = 6, 384, 160
    counts = [3, 0, 17, 1, 40, 5]
    experts, x, offsets = moe_problem(E, K, N, counts, bits, gs, act, seed=bits * 31 + gs)
    xt, qw, qz, sc, gi, off = moe_upload(experts, x, offsets, act, dev)
    T = x.shape[0]
    xt = torch.cat([xt, torch.ones((2, K), dtype=torch.float16, device=dev)])   # 2 rows of no expert
    out = torch.full((T + 2, N), 7.0, dtype=torch.float16, device=dev)
    gq.moe_gemm(xt, qw, qz, sc, gi, off, max(counts), bits, gs, True, out=out)
    ref = oracle.moe_gemm_ref(x, [(L.qweight, L.qzeros, L.scales, L.g_idx) for L in experts], offsets, bits, gs,
                              True, K, N)
    assert_close(out[:T], ref)
    assert bool((out[T:] == 7.0).all())


def test_moe_gemm_bounds(dev):
    """max_tokens_per_expert below an expert's count leaves its extra rows
    untouched; offsets past T are clamped to T (nothing outside x / out)."""
    E, K, N, bits, gs = 3, 256, 96, 4, 128
    counts = [20, 5, 9]
    experts, x, offsets = moe_problem(E, K, N, counts, bits, gs, False, seed=9)
    xt, qw, qz, sc, gi, off = moe_upload(experts, x, offsets, False, dev)
    ref = oracle.moe_gemm_ref(x, [(L.qweight, L.qzeros, L.scales, None) for L in experts], offsets, bits, gs,
                              True, K, N)
    out = torch.full((x.shape[0], N), 7.0, dtype=torch.float16, device=dev)
    gq.moe_gemm(xt, qw, qz, sc, None, off, 16, bits, gs, True, out=out)
    assert_close(out[:16], ref[:16])                 # expert 0: its first 16 rows only
    assert bool((out[16:20] == 7.0).all())
    assert_close(out[20:], ref[20:])
    # offsets running past T: expert 2's rows are clamped to [25, 34)
    off2 = torch.tensor([0, 20, 25, 1000], dtype=torch.int32, device=dev)
    out2 = torch.full((x.shape[0], N), 7.0, dtype=torch.float16, device=dev)
    gq.moe_gemm(xt, qw, qz, sc, None, off2, 1000, bits, gs, True, out=out2)
    assert_close(out2, ref)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("bits,gs,act", [(4, 128, False), (4, 32, False), (3, 128, True), (8, 128, False),
                                         (2, 64, False)])
def test_moe_gemm_paths_parity(dev, path, bits, gs, act):
    """Both grouped kernels on prefill-sized batches: the decode kernel (blocks
    of 16 rows) and the prefill kernel (128-row tiles per expert: several row
    tiles, a partial one, an empty expert, a one-row expert, a column tile
    past N).  Rows of no expert keep their contents."""
    E, K, N = 6, 768, 288
    counts = [130, 0, 37, 200, 1, 64]
    experts, x, offsets = moe_problem(E, K, N, counts, bits, gs, act, seed=bits * 17 + gs + path)
    xt, qw, qz, sc, gi, off = moe_upload(experts, x, offsets, act, dev)
    T = x.shape[0]
    xt = torch.cat([xt, torch.ones((3, K), dtype=torch.float16, device=dev)])
    out = torch.full((T + 3, N), 7.0, dtype=torch.float16, device=dev)
    gq.moe_gemm(xt, qw, qz, sc, gi, off, max(counts), bits, gs, True, out=out, path=path)
    ref = oracle.moe_gemm_ref(x, [(L.qweight, L.qzeros, L.scales, L.g_idx) for L in experts], offsets, bits, gs,
                              True, K, N)
    assert_close(out[:T], ref, f"path {path}")
    assert bool((out[T:] == 7.0).all())


@pytest.mark.parametrize("path", [1, 2])
def test_moe_gemm_row_cap(dev, path):
    """max_tokens_per_expert that is not a multiple of the kernel's row block
    (16) or tile (128): exactly each expert's first 100 rows are computed."""
    E, K, N, bits, gs = 3, 256, 96, 4, 128
    counts = [130, 20, 200]
    experts, x, offsets = moe_problem(E, K, N, counts, bits, gs, False, seed=21 + path)
    xt, qw, qz, sc, gi, off = moe_upload(experts, x, offsets, False, dev)
    ref = oracle.moe_gemm_ref(x, [(L.qweight, L.qzeros, L.scales, None) for L in experts], offsets, bits, gs,
                              True, K, N)
    out = torch.full((x.shape[0], N), 7.0, dtype=torch.float16, device=dev)
    gq.moe_gemm(xt, qw, qz, sc, None, off, 100, bits, gs, True, out=out, path=path)
    done = np.zeros(x.shape[0], dtype=bool)
    for e in range(E):
        done[offsets[e]:offsets[e] + min(100, counts[e])] = True
    rows = torch.from_numpy(np.nonzero(done)[0]).to(dev)
    assert_close(out[rows], ref[done])
    assert bool((out[torch.from_numpy(np.nonzero(~done)[0]).to(dev)] == 7.0).all())


def test_moe_gemm_auto_path(dev):
    """Path 0 runs the decode kernel up to 16 rows per expert and the prefill
    kernel above: bit-identical to the forced path either way."""
    E, K, N, bits, gs = 4, 512, 256, 4, 128
    for counts in ([16, 3, 0, 9], [17, 3, 0, 9]):
        experts, x, offsets = moe_problem(E, K, N, counts, bits, gs, False, seed=33)
        xt, qw, qz, sc, gi, off = moe_upload(experts, x, offsets, False, dev)
        mt = max(counts)
        outs = [gq.moe_gemm(xt, qw, qz, sc, None, off, mt, bits, gs, True, path=p) for p in (0, 1, 2)]
        want = outs[1] if mt <= 16 else outs[2]
        assert torch.equal(outs[0].view(torch.int16), want.view(torch.int16)), counts


def test_moe_gemm_full_size_mixtral(dev):
    """Mixtral-class expert FFN shape (4096 -> 14336, 8 experts, 16 tokens x
    top-2 routing), 4-bit g128: sampled columns against the oracle."""
    E, K, N, bits, gs = 8, 4096, 14336, 4, 128
    rng = np.random.default_rng(5)
    picks = np.array([rng.choice(E, size=2, replace=False) for _ in range(16)]).ravel()
    counts = np.bincount(picks, minlength=E)
    experts, x, offsets = moe_problem(E, K, N, counts, bits, gs, False, seed=11, sym=True, is_v2=False)
    xt, qw, qz, sc, gi, off = moe_upload(experts, x, offsets, False, dev)
    out = gq.moe_gemm(xt, qw, qz, sc, None, off, int(counts.max()), bits, gs, False)
    cols = np.arange(0, N, 149)
    ref = oracle.moe_gemm_ref(x, [(L.qweight, L.qzeros, L.scales, None) for L in experts], offsets, bits, gs,
                              False, K, N, cols=cols)
    assert_close(out[:, torch.from_numpy(cols).to(dev)], ref)


def test_gemm_closed_forms(dev):
    """One-hot rows of x pick rows of W^ (exact up to fp16 output rounding,
    which is the identity for fp16 inputs); x = 0 gives 0."""
    bits, K, N, gs = 4, 256, 128, 64
    d, L = quantized(K, N, 1, bits, gs, False, True, False, seed=3)
    qw, qz, sc, gi = upload(L, dev)
    w_ref = oracle.dequant_ref(L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N)
    x = np.zeros((20, K), dtype=np.float16)
    ks = [0, 1, 31, 32, 63, 64, 100, 127, 128, 129, 200, 255, 7, 8, 9, 15, 16, 17, 250, 40]
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    xt = torch.from_numpy(x).to(dev)
    for p, Ms in ((gq.PATH_DECODE, (1, 16)), (gq.PATH_PREFILL, (20,))):
        for M in Ms:
            y = gq.gemm(xt[:M].contiguous(), qw, qz, sc, gi, bits, gs, True, path=p).cpu().numpy()
            assert np.array_equal(y.view(np.uint16), w_ref[ks[:M]].view(np.uint16)), (p, M)
    y0 = gq.gemm(torch.zeros((5, K), dtype=torch.float16, device=dev), qw, qz, sc, gi, bits, gs, True)
    assert (y0 == 0).all()


def test_gemm_m_zero(dev):
    d, L = quantized(64, 32, 1, 4, 32, False, True, False)
    qw, qz, sc, gi = upload(L, dev)
    y = gq.gemm(torch.zeros((0, 64), dtype=torch.float16, device=dev), qw, qz, sc, gi, 4, 32, True)
    assert tuple(y.shape) == (0, 32)


# ------------------------------------------------------------------ full-size workloads, sampled columns
def workload_cases():
    cases = []
    for name, wl in WORKLOADS.items():
        for layer in wl.layers:
            for M in wl.Ms:
                cases.append(pytest.param(name, layer.name, M, id=f"{name}-{layer.name}-M{M}"))
    return cases


@pytest.mark.parametrize("wname,lname,M", workload_cases())
def test_workload_full_size(dev, wname, lname, M):
    wl = WORKLOADS[wname]
    layer = next(l for l in wl.layers if l.name == lname)
    K, N = layer.K, layer.N
    d = draw_workload_layer(wl, layer, M, seed=0)
    L = oracle.quantize_layer(d.W, wl.bits, wl.group_size, wl.sym, wl.is_v2, d.g_idx)
    if wl.bits == 2 and wl.outlier_rate > 0:
        assert set(np.unique(L.zero)) == {0, 1, 2, 3}
    qw, qz, sc, gi = upload(L, dev)
    # the library's quantizer reproduces the oracle's packed tensors exactly
    gqw, gqz, gsc = gq.quantize(torch.from_numpy(d.W).to(dev), gi, wl.bits, wl.group_size, wl.sym, wl.is_v2)
    assert torch.equal(gqw, qw) and torch.equal(gqz, qz) and torch.equal(gsc.view(torch.int16), sc.view(torch.int16))
    del gqw, gqz, gsc, d.W
    xt = torch.from_numpy(d.x).to(dev)
    y = gq.gemm(xt, qw, qz, sc, gi, wl.bits, wl.group_size, wl.is_v2).cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(1)
    cols = np.unique(np.concatenate([rng.choice(N, 48, replace=False), [0, 1, 2, 3, N - 4, N - 3, N - 2, N - 1]]))
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, wl.bits, wl.group_size, wl.is_v2,
                               K, N, cols=cols)
    assert np.isfinite(y).all()
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.max(np.abs(y[:, cols] - ref))
    assert err <= TOL * rms, f"max err {err:.3e} > {TOL} * rms {rms:.3e}"
    # dequant, bit-exact on the same sampled columns
    w = gq.dequant(qw, qz, sc, gi, wl.bits, wl.group_size, wl.is_v2)[:, torch.from_numpy(cols).to(dev)]
    w_ref = oracle.dequant_ref(L.qweight, L.qzeros, L.scales, L.g_idx, wl.bits, wl.group_size, wl.is_v2, K, N,
                               cols=cols)
    assert np.array_equal(w.cpu().numpy().view(np.uint16), w_ref.view(np.uint16))


# ------------------------------------------------------------------ v1 <-> v2 zero conversion, bit-exact
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("to_v2", [True, False])
def test_convert_zeros_bit_exact(dev, bits, to_v2):
    """gptq_convert_zeros matches the oracle's packed conversion word for word,
    counts the lossy fields, and converts in place."""
    for G, N in ((3, 32), (7, 4128), (1, 96), (200, 1056)):
        qz = random_words(np.random.default_rng(G * 31 + bits), (G, N * bits // 32))
        qz[0, 0], qz[-1, -1] = -1, 0                  # all-max fields, all-zero fields
        want, lossy = oracle.convert_zeros_packed(qz, bits, N, to_v2)
        t = torch.from_numpy(qz).to(dev)
        cnt = torch.zeros(1, dtype=torch.int32, device=dev)
        got = gq.convert_zeros(t, bits, N, to_v2, lossy_count=cnt)
        assert np.array_equal(got.cpu().numpy(), want), (G, N)
        assert int(cnt.item()) == lossy, (G, N)
        assert np.array_equal(t.cpu().numpy(), qz)    # input untouched
        gq.convert_zeros(t, bits, N, to_v2, out=t)    # in place, no counter
        assert np.array_equal(t.cpu().numpy(), want), (G, N, "in place")


def test_convert_zeros_then_gemm_matches_v1(dev):
    """A v1 layer converted to v2 on the GPU gives the same GEMM result as the
    v1 layer read with is_v2 = 0 (dequant compared bit for bit)."""
    K, N, gs, bits = 512, 256, 128, 4
    d = draw_layer(K, N, 1, sigma=0.02, group_size=gs, seed=3)
    L = oracle.quantize_layer(d.W, bits, gs, False, False)
    qw, qz, sc, _ = upload(L, dev)
    qz2 = gq.convert_zeros(qz, bits, N, True)
    w1 = gq.dequant(qw, qz, sc, None, bits, gs, False)
    w2 = gq.dequant(qw, qz2, sc, None, bits, gs, True)
    assert torch.equal(w1.view(torch.int16), w2.view(torch.int16))


# ------------------------------------------------------------------ quantize + pack, bit-exact
QZ_GRID = list(itertools.product(BITS, (False, True), (False, True), (False, True)))


@pytest.mark.parametrize("bits,sym,is_v2,act", QZ_GRID)
def test_quantize_bit_exact(dev, bits, sym, is_v2, act):
    """gptq_quantize reproduces the oracle's min/max quantizer and packers bit for
    bit (codes decided in fp64 on both sides), including degenerate groups and
    groups whose weights all share one sign (the clamped asymmetric zero)."""
    for K, N, gs in ((512, 544, 64), (256, 96, 128), (96, 32, 32)):
        d = draw_layer(K, N, 1, sigma=0.02, group_size=gs, outlier_rate=0.01, act_order=act, seed=bits + K)
        W = d.W.copy()
        W[:, 3] = 0.125                      # constant column: degenerate group -> scale 1
        W[:gs, 5] = 1e-9                     # scale underflows to 0 in fp16 -> 1
        W[:, 7] *= 1e-4                      # fp16-subnormal scales
        W[:, 9] = np.abs(W[:, 9]) + 0.01     # one-signed groups: the asymmetric zero clamps to 0 ...
        W[:, 11] = -np.abs(W[:, 11]) - 0.01  # ... and to 2^b - 1
        L = oracle.quantize_layer(W, bits, gs, sym, is_v2, d.g_idx)
        gi = None if d.g_idx is None else torch.from_numpy(d.g_idx).to(dev)
        qw, qz, sc = gq.quantize(torch.from_numpy(W).to(dev), gi, bits, gs, sym, is_v2)
        assert np.array_equal(qw.cpu().numpy(), L.qweight), (K, N, gs, "qweight")
        assert np.array_equal(qz.cpu().numpy(), L.qzeros), (K, N, gs, "qzeros")
        assert np.array_equal(sc.cpu().numpy().view(np.uint16), L.scales.view(np.uint16)), (K, N, gs, "scales")


# ------------------------------------------------------------------ read ceiling
@pytest.mark.parametrize("nbytes", [0, 16, 8192, 8192 + 48, 3 * 8192 - 16, (1 << 20) + 4096 + 16])
def test_read_ceiling_reads_and_leaves_sink(dev, nbytes):
    """gptq_read_ceiling only reads: on a buffer of repeated words its keep-alive
    store never fires, whatever the ragged length (whole and partial 8 KiB
    workgroup spans), and the buffer is untouched."""
    buf = torch.full(((1 << 20) // 4 + 2048,), 0x3C003C00, dtype=torch.int32, device=dev)
    sink = torch.full((1,), -7, dtype=torch.int32, device=dev)
    gq.read_ceiling(buf, nbytes, sink=sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == -7
    assert bool((buf == 0x3C003C00).all())


def test_read_ceiling_rejects_bad_arguments(dev):
    buf = torch.zeros(1024, dtype=torch.int32, device=dev)
    with pytest.raises(gq.GptqError):
        gq.read_ceiling(buf, 24)                           # not a multiple of 16 bytes
    with pytest.raises(gq.GptqError):
        gq.read_ceiling(buf[2:], 16)                       # not 16-byte aligned
