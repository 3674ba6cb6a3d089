"""Pins for the CPU oracle: each test checks it against something other than itself.

- hand-derived packed words and worked quantization examples (tests/golden);
- an independent pure-Python extractor (one big integer per column);
- Python's own half-precision packing (struct 'e') for fp16 rounding, and
  torch's float32 -> bfloat16 conversion for bfloat16 rounding;
- closed forms and invariants of the min/max formulas and of the v1/v2 zero
  formats ("Enhancing vLLM's support for the GPTQv2 format", sections "Weight
  quantization of LLMs" and "From GPTQv1 to GPTQv2");
- brute-force element-by-element dequant and GEMM on tiny inputs.
"""
import itertools
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
from workload import draw_layer, random_words

BITS = (2, 3, 4, 8)


# ---------------------------------------------------------------- independent helpers
def half_py(v: float) -> float:
    """Round a Python float to fp16 (ties to even) with the standard library."""
    return struct.unpack("<e", struct.pack("<e", v))[0]


def bigint_fields(words_col, bits, L):
    """Fields of one packed column via one Python integer (no numpy shifts)."""
    big = 0
    for r, w in enumerate(words_col):
        big |= (int(w) & 0xFFFFFFFF) << (32 * r)
    return [(big >> (i * bits)) & ((1 << bits) - 1) for i in range(L)]


def bigint_pack(values, bits):
    big = 0
    for i, v in enumerate(values):
        big |= int(v) << (i * bits)
    nwords = len(values) * bits // 32
    return [(big >> (32 * r)) & 0xFFFFFFFF for r in range(nwords)]


def to_i32(u):
    return u - (1 << 32) if u >= (1 << 31) else u


# ---------------------------------------------------------------- fp16 rounding
def test_fp16_rne_matches_struct_half():
    vals = [0.0, -0.0, 1.0, 1 + 2**-11, 1 + 3 * 2**-11, 1 + 2**-10 + 2**-11, 2048 + 1, 2048 + 3,
            65504.0, 65519.0, -65504.0, 2**-24, 2**-25, 3 * 2**-26, 2**-14 - 2**-25,
            6.1e-5, 5.96e-8, 0.1, -0.3, 1e-3, 1234.5678]
    rng = np.random.default_rng(1)
    vals += list(rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 5, 2000))
    vals = [v for v in vals if abs(v) < 65520.0]
    got = oracle.fp16_rne(np.array(vals)).astype(np.float64)
    want = np.array([half_py(v) for v in vals])
    assert np.array_equal(got, want)
    assert np.isinf(oracle.fp16_rne(np.array([65520.0, -1e6]))).all()


# ---------------------------------------------------------------- packing
def test_pack_golden_words(golden_dir):
    with open(os.path.join(golden_dir, "packed_words.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        vals = np.array(c["values"], dtype=np.int64)[:, None]
        want = np.array([to_i32(int(h, 16)) for h in c["words_hex"]], dtype=np.int64)
        packed = oracle.pack_fields(vals, c["bits"])
        assert packed.dtype == np.int32
        assert np.array_equal(packed[:, 0].astype(np.int64), want), c
        back = oracle.unpack_fields(packed, c["bits"], len(c["values"]))
        assert np.array_equal(back[:, 0], vals[:, 0])


@pytest.mark.parametrize("bits", BITS)
def test_pack_unpack_roundtrip_and_edges(bits):
    rng = np.random.default_rng(bits)
    L, C = 96, 12
    qmax = (1 << bits) - 1
    patterns = [
        rng.integers(0, qmax + 1, (L, C)),
        np.zeros((L, C), dtype=np.int64),
        np.full((L, C), qmax),
        np.tile((np.arange(L) % 2 * qmax)[:, None], (1, C)),
        np.tile((np.arange(L) % (qmax + 1))[:, None], (1, C)),
        np.full((L, C), 1 << (bits - 1)),          # top bit of every field set
    ]
    for vals in patterns:
        packed = oracle.pack_fields(vals, bits)
        assert packed.shape == (L * bits // 32, C)
        assert np.array_equal(oracle.unpack_fields(packed, bits, L), vals)


@pytest.mark.parametrize("bits", BITS)
def test_unpack_matches_bigint_extractor(bits):
    rng = np.random.default_rng(100 + bits)
    L = 64
    words = random_words(rng, (L * bits // 32, 5))
    got = oracle.unpack_fields(words, bits, L)
    for c in range(words.shape[1]):
        assert list(got[:, c]) == bigint_fields(words[:, c], bits, L)
    vals = rng.integers(0, 1 << bits, (L, 3))
    packed = oracle.pack_fields(vals, bits)
    for c in range(3):
        assert [to_i32(u) for u in bigint_pack(vals[:, c], bits)] == list(packed[:, c])


@pytest.mark.parametrize("bits", BITS)
def test_pack_along_n_layout(bits):
    """qzeros rows are packed along N: row g's words hold columns 0..N-1 as one stream."""
    rng = np.random.default_rng(7 + bits)
    G, N = 3, 64
    stored = rng.integers(0, 1 << bits, (G, N))
    qz = oracle.pack_along_n(stored, bits)
    assert qz.shape == (G, N * bits // 32) and qz.dtype == np.int32
    for g in range(G):
        assert bigint_fields(qz[g], bits, N) == list(stored[g])
    assert np.array_equal(oracle.unpack_along_n(qz, bits, N), stored)


def test_pack_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.pack_fields(np.zeros((7, 1), dtype=np.int64), 4)      # 28 bits
    with pytest.raises(ValueError):
        oracle.pack_fields(np.full((8, 1), 16), 4)                    # out of range


# ---------------------------------------------------------------- quantizer
def test_quantize_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "minmax_worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        W = np.array(c["w"], dtype=np.float64)[:, None]
        K = W.shape[0]
        q, zero, scale = oracle.quantize_minmax(W, c["bits"], K, c["sym"])
        assert float(scale[0, 0]) == c["scale"], c["name"]
        assert int(zero[0, 0]) == c["zero"], c["name"]
        assert list(q[:, 0]) == c["q"], c["name"]
        assert int(oracle.store_zeros(zero, c["bits"], True)[0, 0]) == c["stored_zero_v2"]
        assert int(oracle.store_zeros(zero, c["bits"], False)[0, 0]) == c["stored_zero_v1"]
        # dequant through the packed path needs K*b % 32 == 0: pad with zero rows
        Kp = K
        while (Kp * c["bits"]) % 32:
            Kp += 1
        qp = np.zeros((Kp, 32), dtype=np.int64)
        qp[:K, 0] = q[:, 0]
        for is_v2, key in ((True, "w_hat"), (False, "w_hat_if_read_as_v1")):
            if key not in c:
                continue
            stored = np.zeros((1, 32), dtype=np.int64)
            stored[0, 0] = oracle.store_zeros(zero, c["bits"], is_v2)[0, 0]
            sc = np.ones((1, 32), dtype=np.float16)
            sc[0, 0] = scale[0, 0]
            w_hat = oracle.dequant_ref(oracle.pack_along_k(qp, c["bits"]),
                                       oracle.pack_along_n(stored, c["bits"]), sc, None,
                                       c["bits"], Kp, is_v2, Kp, 32)
            assert list(w_hat[:K, 0].astype(np.float64)) == c[key], (c["name"], key)


@pytest.mark.parametrize("bits,sym", list(itertools.product(BITS, (False, True))))
def test_quantizer_invariants(bits, sym):
    d = draw_layer(256, 48, 1, sigma=0.02, group_size=64, outlier_rate=0.01, seed=bits)
    q, zero, scale = oracle.quantize_minmax(d.W, bits, 64, sym)
    qmax = (1 << bits) - 1
    assert q.min() >= 0 and q.max() <= qmax
    assert zero.min() >= 0 and zero.max() <= qmax
    if sym:
        assert (zero == (1 << (bits - 1))).all()
        v1 = oracle.store_zeros(zero, bits, False)
        assert (v1 == (1 << (bits - 1)) - 1).all()      # e.g. stored 7 -> runtime 8 at 4-bit
    s = scale.astype(np.float64)
    g = np.arange(256) // 64
    W = d.W.astype(np.float64)
    err = np.abs(W - (q - zero[g]) * s[g])
    clamped = (q == 0) | (q == qmax)
    # round-to-nearest: error <= s/2 wherever the code was not clamped
    assert (err[~clamped] <= s[g][~clamped] / 2 * (1 + 1e-12)).all()
    # clamped codes are group extremes stretched at most by the fp16 rounding of s
    bound = s[g] * (0.5 + qmax * 2.0 ** -11) * (1 + 1e-12)
    assert (err[clamped] <= bound[clamped]).all()


def test_degenerate_group_uses_unit_scale():
    W = np.zeros((64, 4), dtype=np.float32)
    W[:, 1] = 0.25                        # constant column
    q, zero, scale = oracle.quantize_minmax(W, 4, 32, sym=False)
    assert (scale == np.float16(1.0)).all()
    assert (zero == 0).all()
    assert (q[:, 0] == 0).all() and (q[:, 1] == 0).all()   # rint(0.25) = 0


def test_act_order_groups_follow_g_idx():
    d = draw_layer(128, 16, 1, sigma=0.02, group_size=32, act_order=True, seed=3)
    assert sorted(np.bincount(d.g_idx)) == [32] * 4
    q, zero, scale = oracle.quantize_minmax(d.W, 4, 32, sym=False, g_idx=d.g_idx)
    for g in range(4):
        rows = d.g_idx == g
        Wg = d.W[rows].astype(np.float64)
        s = float(half_py((Wg.max(0) - Wg.min(0))[0] / 15))
        assert float(scale[g, 0]) == s


# ---------------------------------------------------------------- v1 / v2 formats
@pytest.mark.parametrize("bits", BITS)
def test_v1_v2_closed_forms(bits):
    d = draw_layer(256, 32, 1, sigma=0.02, group_size=32, outlier_rate=0.02, seed=11)
    q, zero, scale = oracle.quantize_minmax(d.W, bits, 32, sym=False)
    qw = oracle.pack_along_k(q, bits)
    v2 = oracle.store_zeros(zero, bits, True)
    v1 = oracle.store_zeros(zero, bits, False)
    dq = lambda st, is_v2: oracle.dequant_ref(qw, oracle.pack_along_n(st, bits), scale, None,
                                              bits, 32, is_v2, 256, 32)
    w_v2 = dq(v2, True)
    # v1 -> v2 is lossless: stored + 1 read as v2 equals the v1 reading
    w_v1 = dq(v1, False)
    assert np.array_equal(dq(oracle.convert_zeros_v1_to_v2(v1, bits), True).view(np.uint16),
                          w_v1.view(np.uint16))
    # v2 -> v1 changes q - z by exactly -1 in groups whose zero is 0, nowhere else
    g = np.arange(256) // 32
    z0 = (zero == 0)[g]
    s = scale.astype(np.float64)[g]
    assert np.array_equal(w_v1.view(np.uint16)[~z0], w_v2.view(np.uint16)[~z0])
    want = oracle.fp16_rne((q - 1).astype(np.float64) * s)
    assert np.array_equal(w_v1[z0].view(np.uint16), want[z0].view(np.uint16))
    # effective v1 zeros live in [1, 2^b - 1]
    assert (v1 + 1).min() >= 1 and (v1 + 1).max() <= (1 << bits) - 1
    assert np.array_equal(oracle.convert_zeros_v2_to_v1(v2, bits), v1)


def test_int2_v1_zero_range_shrinks():
    z = np.array([[0, 1, 2, 3]])
    v1 = oracle.store_zeros(z, 2, False)
    assert list((v1 + 1)[0]) == [1, 1, 2, 3]     # [0,3] -> [1,3]
    with pytest.raises(ValueError):
        oracle.convert_zeros_v1_to_v2(np.array([[3]]), 2)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("to_v2", [True, False])
def test_convert_zeros_packed_bruteforce(bits, to_v2):
    """Packed conversion against per-field big-integer arithmetic: +1 saturating
    at 2^b - 1 (v1 -> v2) or -1 clamped at 0 (v2 -> v1), every field alone."""
    G, N = 5, 64
    qz = random_words(np.random.default_rng(bits + 10 * to_v2), (G, N * bits // 32))
    qz[0, 0], qz[1, -1] = -1, 0          # a word of all-max fields, a word of zero fields
    out, lossy = oracle.convert_zeros_packed(qz, bits, N, to_v2)
    top = (1 << bits) - 1
    want_lossy = 0
    for g in range(G):
        f = bigint_fields(qz[g], bits, N)
        if to_v2:
            conv = [min(v + 1, top) for v in f]
            want_lossy += sum(v == top for v in f)
        else:
            conv = [max(v - 1, 0) for v in f]
            want_lossy += sum(v == 0 for v in f)
        assert [int(w) & 0xFFFFFFFF for w in out[g]] == bigint_pack(conv, bits)
    assert lossy == want_lossy > 0


@pytest.mark.parametrize("bits", BITS)
def test_convert_zeros_packed_keeps_dequant(bits):
    """A quantizer's v1 zeros converted to v2 dequantize to the same fp16 bits
    when read as v2, and converting back restores the v1 words."""
    d = draw_layer(128, 64, 1, sigma=0.02, group_size=32, outlier_rate=0.02, seed=5)
    lay = oracle.quantize_layer(d.W, bits, 32, sym=False, is_v2=False)
    qz2, lossy = oracle.convert_zeros_packed(lay.qzeros, bits, 64, True)
    assert lossy == 0
    w1 = oracle.dequant_ref(lay.qweight, lay.qzeros, lay.scales, None, bits, 32, False, 128, 64)
    w2 = oracle.dequant_ref(lay.qweight, qz2, lay.scales, None, bits, 32, True, 128, 64)
    assert np.array_equal(w1.view(np.uint16), w2.view(np.uint16))
    back, _ = oracle.convert_zeros_packed(qz2, bits, 64, False)
    assert np.array_equal(back, lay.qzeros)


@pytest.mark.parametrize("bits", BITS)
def test_repack_tiled_index_map(bits):
    """Tiled layout against its element-wise definition, written as loops:
    word (t, c, r, j) = qweight[c*b + r, 16 t + j], except that a 4-bit word
    holds field 2i in nibble i and field 2i + 1 in nibble i + 4 (i < 4; field
    m of checkpoint word is its nibble m, row 32 c + 8 r + m); and the
    inverse."""
    K, N = 96, 48
    qw = random_words(np.random.default_rng(bits), (K * bits // 32, N))
    tiled = oracle.repack_tiled(qw, bits)
    assert tiled.shape == (N // 16, K // 32, bits, 16) and tiled.dtype == np.int32
    for t in range(N // 16):
        for c in range(K // 32):
            for r in range(bits):
                for j in range(16):
                    src = int(qw[c * bits + r, 16 * t + j]) & 0xFFFFFFFF
                    got = int(tiled[t, c, r, j]) & 0xFFFFFFFF
                    if bits != 4:
                        assert got == src
                        continue
                    for i in range(4):
                        assert (got >> (4 * i)) & 15 == (src >> (4 * (2 * i))) & 15
                        assert (got >> (4 * (i + 4))) & 15 == (src >> (4 * (2 * i + 1))) & 15
    assert np.array_equal(oracle.unrepack_tiled(tiled.ravel(), bits, K, N), qw)


def test_moe_gemm_ref_rows_match_their_expert():
    """Each routed row equals that single row through its own expert's layer,
    computed from the dequantized weights with an explicit per-row loop; rows
    of no expert stay NaN."""
    K, N, gs, bits = 64, 32, 32, 4
    experts = []
    for e in range(3):
        d = draw_layer(K, N, 1, sigma=0.02, group_size=gs, seed=40 + e)
        L = oracle.quantize_layer(d.W, bits, gs, False, True)
        experts.append((L.qweight, L.qzeros, L.scales, None))
    x = draw_layer(K, N, 9, sigma=0.02, group_size=gs, seed=50).x
    offsets = [0, 4, 4, 8]                      # expert 1 has no rows; row 8 has no expert
    y = oracle.moe_gemm_ref(x, experts, offsets, bits, gs, True, K, N)
    for e in range(3):
        W = oracle.dequant_ref(*experts[e][:3], None, bits, gs, True, K, N).astype(np.float64)
        for r in range(offsets[e], offsets[e + 1]):
            want = [sum(float(x[r, k]) * W[k, n] for k in range(K)) for n in range(N)]
            assert np.allclose(y[r], want, rtol=0, atol=1e-12)
    assert np.isnan(y[8]).all()


@pytest.mark.parametrize("bits", BITS)
def test_sort_act_order(bits):
    """Sorted rows: packed row fields follow perm (checked field by field with
    big-integer extraction), perm sorts g_idx into i // gs, and the GEMM with
    x[:, perm] on the sorted layer (no g_idx) equals the act-order GEMM."""
    K, N, gs = 256, 64, 64
    d = draw_layer(K, N, 3, sigma=0.02, group_size=gs, act_order=True, seed=bits + 60)
    L = oracle.quantize_layer(d.W, bits, gs, False, True, d.g_idx)
    qs, perm = oracle.sort_act_order(L.qweight, L.g_idx, bits, gs, K)
    assert sorted(perm.tolist()) == list(range(K))
    assert np.array_equal(L.g_idx[perm], np.arange(K) // gs)
    for n in (0, 17, N - 1):
        orig = bigint_fields(L.qweight[:, n], bits, K)
        new = bigint_fields(qs[:, n], bits, K)
        assert new == [orig[p] for p in perm]
    y_act = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N)
    y_srt = oracle.gptq_gemm_ref(d.x[:, perm], qs, L.qzeros, L.scales, None, bits, gs, True, K, N)
    assert np.allclose(y_act, y_srt, rtol=0, atol=1e-12)
    bad = L.g_idx.copy()
    bad[0] = (bad[0] + 1) % (K // gs)           # one group one row short, another one long
    with pytest.raises(ValueError):
        oracle.sort_act_order(L.qweight, bad, bits, gs, K)


# ---------------------------------------------------------------- dequant, brute force
def dequant_bruteforce(qweight, qzeros, scales, g_idx, bits, gs, is_v2, K, N):
    cols = [bigint_fields(qweight[:, n], bits, K) for n in range(N)]
    zrows = [bigint_fields(qzeros[g], bits, N) for g in range(qzeros.shape[0])]
    out = np.empty((K, N), dtype=np.float16)
    for k in range(K):
        g = int(g_idx[k]) if g_idx is not None else k // gs
        for n in range(N):
            z = zrows[g][n] + (0 if is_v2 else 1)
            out[k, n] = half_py((cols[n][k] - z) * float(scales[g, n]))
    return out


@pytest.mark.parametrize("bits,is_v2,act", list(itertools.product(BITS, (False, True), (False, True))))
def test_dequant_matches_bruteforce(bits, is_v2, act):
    K, N, gs = 64, 32, 32
    rng = np.random.default_rng(bits * 10 + is_v2 * 2 + act)
    qweight = random_words(rng, (K * bits // 32, N))
    qzeros = random_words(rng, (K // gs, N * bits // 32))
    scales = (rng.standard_normal((K // gs, N)) * 0.02).astype(np.float16)
    scales[0, 0] = np.float16(6e-8)           # products land in the fp16 subnormal range
    g_idx = rng.permutation(np.arange(K) // gs).astype(np.int32) if act else None
    got = oracle.dequant_ref(qweight, qzeros, scales, g_idx, bits, gs, is_v2, K, N)
    want = dequant_bruteforce(qweight, qzeros, scales, g_idx, bits, gs, is_v2, K, N)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_dequant_v1_max_zero_does_not_wrap():
    """A v1 stored zero of 2^b - 1 means z = 2^b, never 0."""
    bits, K, N = 8, 32, 32
    qweight = np.zeros((K * bits // 32, N), dtype=np.int32)
    qzeros = oracle.pack_along_n(np.full((1, N), 255), bits)
    scales = np.ones((1, N), dtype=np.float16)
    w = oracle.dequant_ref(qweight, qzeros, scales, None, bits, K, False, K, N)
    assert (w == np.float16(-256.0)).all()


# ---------------------------------------------------------------- GEMM, brute force + closed forms
@pytest.mark.parametrize("bits,is_v2,act", list(itertools.product(BITS, (False, True), (False, True))))
def test_gemm_matches_triple_loop(bits, is_v2, act):
    M, K, N, gs = 3, 64, 32, 32
    d = draw_layer(K, N, M, sigma=0.02, group_size=gs, act_order=act, seed=5)
    L = oracle.quantize_layer(d.W, bits, gs, sym=False, is_v2=is_v2, g_idx=d.g_idx)
    y = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, is_v2, K, N)
    w = dequant_bruteforce(L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, is_v2, K, N)
    for m in range(M):
        for n in range(N):
            exact = math.fsum(float(d.x[m, k]) * float(w[k, n]) for k in range(K))
            assert abs(y[m, n] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_gemm_closed_forms():
    bits, K, N, gs = 4, 128, 64, 32
    d = draw_layer(K, N, 4, sigma=0.02, group_size=gs, seed=9)
    L = oracle.quantize_layer(d.W, bits, gs, sym=False, is_v2=True)
    w = oracle.dequant_ref(L.qweight, L.qzeros, L.scales, None, bits, gs, True, K, N)
    # one-hot rows select rows of W^
    x = np.zeros((3, K), dtype=np.float16)
    for i, k in enumerate((0, 77, K - 1)):
        x[i, k] = 1.0
    y = oracle.gemm_ref(x, w)
    assert np.array_equal(y, w[[0, 77, K - 1]].astype(np.float64))
    assert (oracle.gemm_ref(np.zeros((2, K), np.float16), w) == 0).all()
    # q == z everywhere -> zero output
    zq = np.full((K, N), 5)
    wz = oracle.dequant_ref(oracle.pack_along_k(zq, bits), oracle.pack_along_n(np.full((K // gs, N), 5), bits),
                            L.scales, None, bits, gs, True, K, N)
    assert (oracle.gemm_ref(d.x, wz) == 0).all()
    # s = 1, z = 0, integer x -> exact integer products
    rng = np.random.default_rng(2)
    qi = rng.integers(0, 16, (K, N))
    wi = oracle.dequant_ref(oracle.pack_along_k(qi, bits), oracle.pack_along_n(np.zeros((K // gs, N), int), bits),
                            np.ones((K // gs, N), np.float16), None, bits, gs, True, K, N)
    xi = rng.integers(-3, 4, (2, K)).astype(np.float16)
    assert np.array_equal(oracle.gemm_ref(xi, wi), xi.astype(np.int64) @ qi)


# ---------------------------------------------------------------- bfloat16 activations
def bf16_torch(values):
    """Round float32-exact values to bfloat16 with torch's own conversion."""
    import torch
    t = torch.from_numpy(np.asarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_rne_closed_forms():
    r = oracle.bf16_rne
    one = 1.0
    assert r(np.array([one + 2.0 ** -8]))[0] == one                        # tie -> even
    assert r(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6        # tie -> even (up)
    assert r(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 2.0 ** -7
    assert r(np.array([2.0 ** -133]))[0] == 2.0 ** -133                     # smallest subnormal
    assert r(np.array([2.0 ** -134]))[0] == 0.0                             # tie -> even zero
    assert r(np.array([3 * 2.0 ** -134]))[0] == 2.0 ** -132                 # 1.5 ulp -> 2 ulp
    assert r(np.array([-(2.0 ** -126) * 1.00390625]))[0] == -(2.0 ** -126)  # normal, tie to even
    big = float.fromhex("0x1.fep127")
    assert r(np.array([big]))[0] == big
    assert r(np.array([big + 2.0 ** 118]))[0] == big                          # below the tie at max
    assert np.isinf(r(np.array([big + 2.0 ** 119, -1e39]))).all()          # the tie at max overflows
    assert r(np.array([0.0]))[0] == 0.0 and np.isnan(r(np.array([np.nan])))[0]
    # the bit helpers agree with the format's layout: sign, 8 exponent, 7 mantissa bits
    assert oracle.bf16_bits(np.array([1.0, -2.0, 2.0 ** -133])).tolist() == [0x3F80, 0xC000, 0x0001]
    assert oracle.bf16_from_bits(np.array([0x3F80, 0x4049])).tolist() == [1.0, 3.140625]


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(11)
    v = rng.standard_normal(200000).astype(np.float32)
    with np.errstate(over="ignore"):
        v = (v * np.exp2(rng.integers(-140, 129, v.size)).astype(np.float32)).astype(np.float32)
    # exact ties (8 significant bits + a half ulp)
    t = (rng.integers(128, 256, 2000) * 2 + 1).astype(np.float64) * np.exp2(rng.integers(-20, 20, 2000) - 9)
    vals = np.concatenate([v.astype(np.float64), t, -t])
    assert np.array_equal(oracle.bf16_rne(vals), bf16_torch(vals.astype(np.float32)), equal_nan=True)


@pytest.mark.parametrize("bits,is_v2,act", list(itertools.product(BITS, (False, True), (False, True))))
def test_dequant_bf16_matches_bruteforce(bits, is_v2, act):
    K, N, gs = 64, 32, 32
    rng = np.random.default_rng(bits * 10 + is_v2 * 2 + act + 100)
    qweight = random_words(rng, (K * bits // 32, N))
    qzeros = random_words(rng, (K // gs, N * bits // 32))
    scales = bf16_torch(rng.standard_normal((K // gs, N)) * 0.02)
    scales[0, 0] = 2.0 ** -130                # products land in the bf16 subnormal range
    g_idx = rng.permutation(np.arange(K) // gs).astype(np.int32) if act else None
    got = oracle.dequant_ref(qweight, qzeros, scales, g_idx, bits, gs, is_v2, K, N, act="bf16")
    cols = [bigint_fields(qweight[:, n], bits, K) for n in range(N)]
    zrows = [bigint_fields(qzeros[g], bits, N) for g in range(K // gs)]
    exact = np.empty((K, N))
    for k in range(K):
        g = int(g_idx[k]) if g_idx is not None else k // gs
        for n in range(N):
            exact[k, n] = (cols[n][k] - zrows[g][n] - (0 if is_v2 else 1)) * float(scales[g, n])
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)   # exact in fp32
    assert np.array_equal(got, bf16_torch(exact))


def test_dequant_bf16_rejects_inexact_scales():
    K, N, bits = 32, 32, 4
    qw = np.zeros((K * bits // 32, N), np.int32)
    qz = np.zeros((1, N * bits // 32), np.int32)
    with pytest.raises(ValueError):
        oracle.dequant_ref(qw, qz, np.full((1, N), 1.0 + 2.0 ** -10), None, bits, K, True, K, N, act="bf16")


def test_gemm_bf16_matches_triple_loop():
    M, K, N, gs, bits = 3, 64, 32, 32, 3
    d = draw_layer(K, N, M, sigma=0.02, group_size=gs, act_order=True, seed=6)
    L = oracle.quantize_layer(d.W, bits, gs, sym=False, is_v2=True, g_idx=d.g_idx)
    s16 = bf16_torch(L.scales.astype(np.float64))
    x16 = bf16_torch(d.x.astype(np.float64))
    y = oracle.gptq_gemm_ref(x16, L.qweight, L.qzeros, s16, L.g_idx, bits, gs, True, K, N, act="bf16")
    cols = [bigint_fields(L.qweight[:, n], bits, K) for n in range(N)]
    zrows = [bigint_fields(L.qzeros[g], bits, N) for g in range(K // gs)]
    for m in range(M):
        for n in range(N):
            w = [bf16_torch([(cols[n][k] - zrows[int(L.g_idx[k])][n]) * float(s16[int(L.g_idx[k]), n])])[0]
                 for k in range(K)]
            exact = math.fsum(float(x16[m, k]) * w[k] for k in range(K))
            assert abs(y[m, n] - exact) <= 1e-12 * max(1.0, abs(exact))


# ---------------------------------------------------------------- the low-bit workload
def test_lowbit_workload_zeros_span_full_range():
    """2-bit g64 asymmetric with 0.5% x10 outliers: stored zeros hit every value 0..3."""
    d = draw_layer(4096, 1024, 1, sigma=0.02, group_size=64, outlier_rate=0.005, seed=0)
    _, zero, _ = oracle.quantize_minmax(d.W, 2, 64, sym=False)
    assert set(np.unique(zero)) == {0, 1, 2, 3}


def test_workload_draws_are_seeded():
    a = draw_layer(256, 64, 2, sigma=0.02, group_size=64, act_order=True, seed=0)
    b = draw_layer(256, 64, 5, sigma=0.02, group_size=64, act_order=True, seed=0)
    assert np.array_equal(a.W, b.W) and np.array_equal(a.g_idx, b.g_idx)
    assert a.x.dtype == np.float16 and a.W.dtype == np.float32
