"""GPU parity for bfloat16 activations (gptq_gemm_bf16, gptq_dequant_bf16) against the oracle.

- gptq_dequant_bf16 must match oracle.dequant_ref(act="bf16") bit for bit;
- gptq_gemm_bf16 must satisfy, element by element,
      |y - y_ref| <= 5e-3 * rms(y_ref) + 2^-8 * |y_ref|
  with y_ref = x . W^ in fp64: the GEMM bar of the fp16 path plus the output's
  own bfloat16 rounding (at most half an ulp, 2^-9 relative, doubled for
  accumulation-order effects at a rounding boundary).

Layers come from the fp16 recipe (seeded draws, quantized by the oracle); x and
the scales are then rounded to bfloat16 by torch's conversion, and the oracle
reads back exactly those bfloat16 values.
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
OUT_ROUND = 2.0 ** -8


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.library()
    return torch.device("cuda:0")


def bf16(a):
    """(bfloat16 CPU tensor, its exact values as float64) of a float array."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(torch.bfloat16)
    return t, t.to(torch.float64).numpy()


def layer_bf16(K, N, M, bits, gs, sym, is_v2, act, seed=0, sigma=0.02):
    d = draw_layer(K, N, M, sigma=sigma, group_size=gs, act_order=act, seed=seed)
    L = oracle.quantize_layer(d.W, bits, gs, sym, is_v2, d.g_idx)
    sc_t, sc = bf16(L.scales.astype(np.float32))
    x_t, x = bf16(d.x.astype(np.float32))
    return L, sc_t, sc, x_t, x


def upload(L, sc_t, dev):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t(L.qweight), t(L.qzeros), sc_t.to(dev), None if L.g_idx is None else t(L.g_idx)


def assert_close_bf16(y_gpu, y_ref, what=""):
    assert y_gpu.dtype == torch.bfloat16
    y = y_gpu.to(torch.float64).cpu().numpy()
    assert np.isfinite(y).all(), what
    rms = np.sqrt(np.mean(y_ref ** 2))
    excess = np.abs(y - y_ref) - (TOL * rms + OUT_ROUND * np.abs(y_ref))
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[i] <= 0, (f"{what}: |y - y_ref| = {abs(y[i] - y_ref[i]):.3e} at {i} exceeds "
                            f"{TOL} * rms {rms:.3e} + 2^-8 * |y_ref| {abs(y_ref[i]):.3e}")


# ------------------------------------------------------------------ dequant, bit-exact
@pytest.mark.parametrize("bits,is_v2,act,gs", list(itertools.product(BITS, (False, True), (False, True), (32, 128))))
def test_dequant_bf16_bit_exact(dev, bits, is_v2, act, gs):
    K, N = 256, 160
    L, sc_t, sc, _, _ = layer_bf16(K, N, 1, bits, gs, False, is_v2, act, seed=bits + 7 * gs)
    qw, qz, sct, gi = upload(L, sc_t, dev)
    w = gq.dequant(qw, qz, sct, gi, bits, gs, is_v2)
    torch.cuda.synchronize()
    assert w.dtype == torch.bfloat16
    ref = oracle.dequant_ref(L.qweight, L.qzeros, sc, L.g_idx, bits, gs, is_v2, K, N, act="bf16")
    assert np.array_equal(w.view(torch.int16).cpu().numpy().view(np.uint16), oracle.bf16_bits(ref))


def _dequant_random(dev, bits, is_v2, special, seed):
    K, N, gs = 128, 96, 32
    rng = np.random.default_rng(seed)
    qweight = random_words(rng, (K * bits // 32, N))
    qzeros = random_words(rng, (K // gs, N * bits // 32))
    sc_t, _ = bf16(rng.standard_normal((K // gs, N)) * 0.02)
    sc_t[0, :len(special)] = torch.tensor(special, dtype=torch.float64).to(torch.bfloat16)
    sc_t[1, :len(special)] = -sc_t[0, :len(special)]
    sc = sc_t.to(torch.float64).numpy()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    w = gq.dequant(t(qweight), t(qzeros), sc_t.to(dev), None, bits, gs, is_v2)
    ref = oracle.dequant_ref(qweight, qzeros, sc, None, bits, gs, is_v2, K, N, act="bf16")
    got = w.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.isfinite(ref).all()
    assert np.array_equal(got, oracle.bf16_bits(ref))


@pytest.mark.parametrize("bits,is_v2", list(itertools.product(BITS, (False, True))))
def test_dequant_bf16_random_words_and_subnormals(dev, bits, is_v2):
    """Every field value, zeros up to 2^b - 1 (2^b under v1), and scales whose
    products fall in the bfloat16 subnormal range (fp32 denormals on the GPU)."""
    _dequant_random(dev, bits, is_v2, [2.0 ** -130, 2.0 ** -133, 2.0 ** -126, 1e-38, 3 * 2.0 ** -131, 0.0, 1.0],
                    40 + bits + is_v2)


@pytest.mark.parametrize("bits,is_v2", list(itertools.product(BITS, (False, True))))
def test_dequant_bf16_large_scales(dev, bits, is_v2):
    """Scales up to the documented bound |s| < 2^119 (so that z s stays finite
    in fp32): the products stay exact up to 2^127."""
    _dequant_random(dev, bits, is_v2, [2.0 ** 118, 1.5 * 2.0 ** 118, 2.0 ** 100, 65504.0, 1e30], 60 + bits + is_v2)


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("bits,is_v2,act,gs", list(itertools.product(BITS, (False, True), (False, True), (32, 128))))
def test_gemm_bf16_small_grid(dev, bits, is_v2, act, gs):
    K, N = 512, 160
    for sym in (False, True):
        L, sc_t, sc, x_t, x = layer_bf16(K, N, 40, bits, gs, sym, is_v2, act, seed=bits * 11 + gs)
        qw, qz, sct, gi = upload(L, sc_t, dev)
        xt = x_t.to(dev)
        for M in (1, 2, 4, 5, 16, 17, 40):
            ref = oracle.gptq_gemm_ref(x[:M], L.qweight, L.qzeros, sc, L.g_idx, bits, gs, is_v2, K, N, act="bf16")
            paths = [gq.PATH_AUTO, gq.PATH_PREFILL] + ([gq.PATH_DECODE] if M <= 16 else [])
            for p in paths:
                y = gq.gemm(xt[:M].contiguous(), qw, qz, sct, gi, bits, gs, is_v2, path=p)
                assert_close_bf16(y, ref, f"M={M} path={p} sym={sym}")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,N,gs", [(96, 32, 32), (288, 224, 96), (256, 64, 16), (1024, 32, 1024)])
def test_gemm_bf16_ragged_and_group_shapes(dev, bits, K, N, gs):
    L, sc_t, sc, x_t, x = layer_bf16(K, N, 33, bits, gs, False, True, False, seed=K + N + gs)
    qw, qz, sct, gi = upload(L, sc_t, dev)
    xt = x_t.to(dev)
    for M in (1, 7, 16, 33):
        ref = oracle.gptq_gemm_ref(x[:M], L.qweight, L.qzeros, sc, None, bits, gs, True, K, N, act="bf16")
        for p in ([gq.PATH_DECODE] if M <= 16 else []) + [gq.PATH_PREFILL]:
            y = gq.gemm(xt[:M].contiguous(), qw, qz, sct, gi, bits, gs, True, path=p)
            assert_close_bf16(y, ref, f"M={M} path={p}")


@pytest.mark.parametrize("bits,M,K,N", [(4, 1, 8192, 512), (3, 4, 8192, 96), (8, 16, 4096, 256), (2, 2, 12288, 64),
                                        (4, 40, 4096, 512), (8, 100, 4096, 256)])
def test_gemm_bf16_long_k(dev, bits, M, K, N):
    """K long enough for several decode phases and (narrow N) split K, whose
    last workgroup writes the bfloat16 result; at M = 40 and 100 the prefill
    kernels split K and the sum kernel writes it."""
    L, sc_t, sc, x_t, x = layer_bf16(K, N, M, bits, 128, False, True, False, seed=K + M)
    qw, qz, sct, gi = upload(L, sc_t, dev)
    ref = oracle.gptq_gemm_ref(x, L.qweight, L.qzeros, sc, None, bits, 128, True, K, N, act="bf16")
    y1 = gq.gemm(x_t.to(dev), qw, qz, sct, gi, bits, 128, True)
    y2 = gq.gemm(x_t.to(dev), qw, qz, sct, gi, bits, 128, True)
    desc = gq.describe(x_t.to(dev), qw, qz, sct, gi, bits, 128, True)
    if M > 16:
        assert desc.startswith("gptq::prefill_bf16") and int(desc.split("k_splits=")[1].split()[0]) > 1, desc
    assert_close_bf16(y1, ref, desc)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))           # deterministic


def test_gemm_bf16_wide_range_activations(dev):
    """x entries far outside fp16's range (their bit patterns would be fp16
    NaNs and infinities) and tiny ones: bfloat16 keeps fp32's exponent range,
    and the kernels move x as raw 16-bit values."""
    K, N, bits, gs = 256, 64, 4, 64
    L, sc_t, sc, _, _ = layer_bf16(K, N, 20, bits, gs, False, True, False, seed=3)
    rng = np.random.default_rng(5)
    xv = rng.standard_normal((20, K)) * np.exp2(rng.integers(-60, 60, (20, K)))
    xv[0, :4] = [2.0 ** 121, -(2.0 ** 120) * 1.5, 2.0 ** -130, 65536.0]
    x_t, x = bf16(xv)
    qw, qz, sct, gi = upload(L, sc_t, dev)
    for M in (1, 16, 20):
        ref = oracle.gptq_gemm_ref(x[:M], L.qweight, L.qzeros, sc, None, bits, gs, True, K, N, act="bf16")
        for p in ([gq.PATH_DECODE] if M <= 16 else []) + [gq.PATH_PREFILL]:
            y = gq.gemm(x_t[:M].contiguous().to(dev), qw, qz, sct, gi, bits, gs, True, path=p)
            yv = y.to(torch.float64).cpu().numpy()
            # per row: the rms of the row sets the scale (rows differ by up to 2^120)
            for m in range(M):
                rms = np.sqrt(np.mean(ref[m] ** 2))
                bound = TOL * rms + OUT_ROUND * np.abs(ref[m])
                assert (np.abs(yv[m] - ref[m]) <= bound).all(), f"M={M} path={p} row {m}"


def test_gemm_bf16_rejects_mixed_types(dev):
    L, sc_t, sc, x_t, x = layer_bf16(128, 32, 2, 4, 32, False, True, False)
    qw, qz, sct, gi = upload(L, sc_t, dev)
    with pytest.raises(ValueError):
        gq.gemm(x_t.to(dev).half(), qw, qz, sct, gi, 4, 32, True)          # fp16 x, bf16 scales
    with pytest.raises(ValueError):
        gq.gemm(x_t.to(dev), qw, qz, sct.half(), gi, 4, 32, True)          # bf16 x, fp16 scales


@pytest.mark.parametrize("bits,is_v2,act,gs", list(itertools.product(BITS, (False, True), (False, True), (32, 128))))
def test_gemm_bf16_tiled_layout(dev, bits, is_v2, act, gs):
    """gptq_gemm_tiled_bf16: the tiled qweight layout (4-bit words in pair
    order) through the bfloat16 decode and prefill kernels, against the oracle
    on the checkpoint arrays."""
    K, N = 512, 160
    L, sc_t, sc, x_t, x = layer_bf16(K, N, 40, bits, gs, False, is_v2, act, seed=bits * 13 + gs + 5 * act)
    qw, qz, sct, gi = upload(L, sc_t, dev)
    qwt = gq.repack_tiled(qw, bits)
    xt = x_t.to(dev)
    for M in (1, 4, 16, 17, 40):
        ref = oracle.gptq_gemm_ref(x[:M], L.qweight, L.qzeros, sc, L.g_idx, bits, gs, is_v2, K, N, act="bf16")
        for p in ([gq.PATH_DECODE] if M <= 16 else []) + [gq.PATH_PREFILL]:
            y = gq.gemm(xt[:M].contiguous(), qwt, qz, sct, gi, bits, gs, is_v2, path=p)
            assert_close_bf16(y, ref, f"tiled M={M} path={p}")


def test_gemm_bf16_describe_names_the_bf16_kernels(dev):
    L, sc_t, sc, x_t, x = layer_bf16(256, 256, 64, 4, 128, True, False, False)
    qw, qz, sct, gi = upload(L, sc_t, dev)
    xt = x_t.to(dev)
    assert gq.describe(xt[:1].contiguous(), qw, qz, sct, gi, 4, 128, False).startswith("gptq::decode_bf16_kernel<4, 1,")
    assert gq.describe(xt, qw, qz, sct, gi, 4, 128, False).startswith("gptq::prefill_bf16_small_kernel<4, false, true, false, 64>")
    x2 = torch.cat([xt, xt]).contiguous()          # 128 rows: the 128-row tile
    assert gq.describe(x2, qw, qz, sct, gi, 4, 128, False).startswith("gptq::prefill_bf16_kernel<4, false, true>")
    qwt = gq.repack_tiled(qw, 4)
    assert gq.describe(xt[:1].contiguous(), qwt, qz, sct, gi, 4, 128, False).startswith("gptq::decode_bf16_kernel<4,")
    assert gq.describe(xt, qwt, qz, sct, gi, 4, 128, False).startswith("gptq::prefill_bf16_small_kernel<4, false, true, true, 64>")


# ------------------------------------------------------------------ full-size layers, sampled columns
@pytest.mark.parametrize("wname,lname,M,tiled", [("llama7b_decode_w4g128", "qkv", 1, False),
                                                 ("llama7b_decode_w4g128", "down", 1, False),
                                                 ("llama7b_decode_w4g128", "gate_up", 1, True),
                                                 ("actorder_decode_w3g128", "up", 16, False),
                                                 ("mlp70b_prefill_w4g128", "up", 2048, False),
                                                 ("mlp70b_prefill_w4g128", "down", 2048, True)])
def test_gemm_bf16_full_size(dev, wname, lname, M, tiled):
    wl = WORKLOADS[wname]
    layer = next(l for l in wl.layers if l.name == lname)
    K, N = layer.K, layer.N
    d = draw_workload_layer(wl, layer, M, seed=0)
    L = oracle.quantize_layer(d.W, wl.bits, wl.group_size, wl.sym, wl.is_v2, d.g_idx)
    del d.W
    sc_t, sc = bf16(L.scales.astype(np.float32))
    x_t, x = bf16(d.x.astype(np.float32))
    qw, qz, sct, gi = upload(L, sc_t, dev)
    if tiled:
        qw = gq.repack_tiled(qw, wl.bits)
    y = gq.gemm(x_t.to(dev), qw, qz, sct, gi, wl.bits, wl.group_size, wl.is_v2)
    rng = np.random.default_rng(2)
    cols = np.unique(np.concatenate([rng.choice(N, 40, replace=False), [0, 1, N - 2, N - 1]]))
    ref = oracle.gptq_gemm_ref(x, L.qweight, L.qzeros, sc, L.g_idx, wl.bits, wl.group_size, wl.is_v2, K, N,
                               cols=cols, act="bf16")
    assert_close_bf16(y[:, torch.from_numpy(cols).to(dev)], ref, f"{wname} {lname} M={M}")
