"""Reference GPTQ quantize / pack / dequant / GEMM in numpy (fp64) -- test infrastructure.

Citations name the page and the section they follow:

[P1-WQ]  "Enhancing vLLM's support for the GPTQv2 format: analysis and
         implementation" (xxxxyu blog), section "Weight quantization of LLMs":
         scale = (wmax - wmin)/(2^b - 1); zero = -round(wmin/scale);
         wq = clamp(round(wo/scale) + zero); dequant w^ = (wq - zero)*scale;
         symmetric groups assume wmax = -wmin, so zero = round((2^b - 1)/2).
[P1-V2]  same page, section "From GPTQv1 to GPTQv2": GPTQv1 stores
         clamp(zero - 1) and adds 1 at run time; GPTQv2 stores zero as is;
         v1 -> v2 is lossless, v2 -> v1 clamps 0 - 1 to 0.
[P1-ADJ] same page, section "Adjustment details": the kernel adds
         zero_offset = (use_v2_format ? 0 : 1) to every unpacked zero; one
         128-bit load carries four adjacent output columns, each with its own
         zero, and the dequantized fp16 rows have stride N.

Readings where the pages are silent (each listed in the design notes):
- round() is round-half-to-even (numpy.rint);
- clamp() bounds are the b-bit unsigned range [0, 2^b - 1]; the asymmetric zero
  is clamped to that range too;
- the scale is computed in fp64 and stored as fp16 (round to nearest even);
  the quantizer then uses the stored fp16 scale; a stored scale of 0
  (degenerate group) is replaced by 1.0;
- symmetric: wabs = max|w| read as wmax = wabs, wmin = -wabs;
- an empty group (possible only with a hand-made g_idx) behaves as all-zero;
- packing: each column's (qweight) or each group row's (qzeros) values form one
  LSB-first bitstream of b-bit fields; word r holds bits [32r, 32r+32).  For
  3-bit, a 32-value chunk spans three words and fields 10 and 21 straddle a
  word boundary.  The int32 words are plain bit containers (logical shifts);
- qweight is [K*b/32, N] (packed along K), qzeros is [G, N*b/32] (packed along
  N), scales is fp16 [G, N], g_idx[k] is the group of row k (absent: k // gs);
- dequant is one round-to-nearest-even of the exact product (q - z)*s to fp16;
- the GEMM is y = x @ W^ with x and W^ widened to fp64;
- bfloat16 activations (named beside fp16 by "Weight-only INT4 quantization:
  GPTQ, AWQ and the Marlin kernel", section 1.2, which gives no formula for
  them): x, the scales and W^ are bfloat16, W^ = bf16_RNE((q - z) * s), the
  same one rounding as the fp16 formula with the other 16-bit type.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

_U32 = np.uint64(0xFFFFFFFF)


def fp16_rne(a) -> np.ndarray:
    """Round fp64 values to fp16, nearest-even; subnormals kept, overflow -> inf.

    numpy converts float64 to float16 directly (one rounding), which is the
    rounding the dequant formula needs [P1-WQ].  Overflow to inf is the
    intended result, so numpy's overflow warning is silenced."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float16)


_BF16_MAX = float.fromhex("0x1.fep127")    # largest finite bfloat16, (2 - 2^-7) 2^127


def bf16_rne(a) -> np.ndarray:
    """Round fp64 values to bfloat16 (8 significant bits, fp32's exponent range),
    nearest-even; subnormals kept, overflow -> inf.  Returns the rounded values
    as float64 (every bfloat16 value is exact there).

    The 16-bit activation type the pages allow besides fp16 ("Weight-only INT4
    quantization: GPTQ, AWQ and the Marlin kernel", section 1.2).  A value with
    |a| in [2^(e-1), 2^e) has bf16 spacing 2^(e-8); below the smallest normal
    2^-126 the spacing stays 2^-133."""
    a = np.asarray(a, dtype=np.float64)
    out = a.copy()
    fin = np.isfinite(a) & (a != 0)
    v = a[fin]
    _, e = np.frexp(v)
    step = np.maximum(e, -125) - 8
    r = np.ldexp(np.rint(np.ldexp(v, -step)), step)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_bits(values) -> np.ndarray:
    """bfloat16 values (float, exactly representable) -> their 16-bit patterns."""
    v = np.asarray(values, dtype=np.float64)
    if not np.array_equal(bf16_rne(v), v, equal_nan=True):
        raise ValueError("values are not exact bfloat16 values")
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    """16-bit bfloat16 patterns -> float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def max_q(bits: int) -> int:
    """Largest b-bit unsigned value, 2^b - 1 [P1-WQ]."""
    return (1 << bits) - 1


def num_groups(K: int, group_size: int) -> int:
    if group_size <= 0 or K % group_size != 0:
        raise ValueError("K must be a positive multiple of group_size")
    return K // group_size


def group_of_rows(K: int, group_size: int, g_idx: Optional[np.ndarray]) -> np.ndarray:
    """Group index of every row k: g_idx[k] when given, else k // group_size."""
    if g_idx is None:
        return np.arange(K, dtype=np.int64) // group_size
    g = np.asarray(g_idx, dtype=np.int64)
    if g.shape != (K,):
        raise ValueError("g_idx must have shape [K]")
    return g


def quantize_minmax(W: np.ndarray, bits: int, group_size: int, sym: bool,
                    g_idx: Optional[np.ndarray] = None):
    """Round-to-nearest min/max quantization of W [K, N] per (group, column) [P1-WQ].

    Returns (q int64 [K,N], zero int64 [G,N], scale fp16 [G,N]); ``zero`` is the
    true zero point, before any storage format is applied."""
    K, N = W.shape
    G = num_groups(K, group_size)
    groups = group_of_rows(K, group_size, g_idx)
    if groups.size and (groups.min() < 0 or groups.max() >= G):
        raise ValueError("g_idx entries must lie in [0, G)")
    qmax = max_q(bits)
    W64 = np.asarray(W, dtype=np.float64)

    q = np.zeros((K, N), dtype=np.int64)
    zero = np.zeros((G, N), dtype=np.int64)
    scale = np.zeros((G, N), dtype=np.float16)
    for g in range(G):
        rows = np.nonzero(groups == g)[0]
        Wg = W64[rows] if rows.size else np.zeros((1, N))
        if sym:
            wabs = np.max(np.abs(Wg), axis=0)
            wmax, wmin = wabs, -wabs
        else:
            wmax = np.max(Wg, axis=0)
            wmin = np.min(Wg, axis=0)
        # scale = (wmax - wmin) / (2^b - 1), stored as fp16
        s16 = fp16_rne((wmax - wmin) / qmax)
        s16 = np.where(s16 == 0, np.float16(1.0), s16)
        s = s16.astype(np.float64)
        if sym:
            # zero = round((2^b - 1) / 2), a constant
            z = np.full(N, np.rint(qmax / 2.0))
        else:
            # zero = -round(wmin / scale), clamped to the b-bit range
            z = np.clip(-np.rint(wmin / s), 0, qmax)
        if rows.size:
            # wq = clamp(round(w / scale) + zero)
            q[rows] = np.clip(np.rint(W64[rows] / s) + z, 0, qmax).astype(np.int64)
        zero[g] = z.astype(np.int64)
        scale[g] = s16
    return q, zero, scale


def store_zeros(zero: np.ndarray, bits: int, is_v2: bool) -> np.ndarray:
    """Zero points as a checkpoint stores them [P1-V2]: v2 keeps zero, v1 keeps
    clamp(zero - 1)."""
    zero = np.asarray(zero, dtype=np.int64)
    if is_v2:
        return zero.copy()
    return np.clip(zero - 1, 0, max_q(bits))


def convert_zeros_v1_to_v2(stored_v1: np.ndarray, bits: int, saturate: bool = False) -> np.ndarray:
    """v1 -> v2: the runtime +1 becomes part of the stored value [P1-V2].  Exact
    for every v1 value a quantizer writes (those are <= 2^b - 2).  A v1 field
    of 2^b - 1 has no v2 encoding: an error, or 2^b - 1 with saturate=True."""
    out = np.asarray(stored_v1, dtype=np.int64) + 1
    if out.size and out.max() > max_q(bits):
        if not saturate:
            raise ValueError("a v1 zero of 2^b - 1 has no v2 encoding")
        out = np.minimum(out, max_q(bits))
    return out


def convert_zeros_v2_to_v1(stored_v2: np.ndarray, bits: int) -> np.ndarray:
    """v2 -> v1: store clamp(zero - 1); a zero of 0 becomes 1 at run time [P1-V2]."""
    return np.clip(np.asarray(stored_v2, dtype=np.int64) - 1, 0, max_q(bits))


def pack_fields(vals: np.ndarray, bits: int) -> np.ndarray:
    """Pack vals [L, C] (each in [0, 2^b)) along axis 0 into int32 words [L*b/32, C].

    Field i of every column sits at bits [i*b, i*b + b) of that column's
    LSB-first bitstream; word r holds stream bits [32r, 32r + 32)."""
    L, C = vals.shape
    if (L * bits) % 32 != 0:
        raise ValueError("L * bits must be a multiple of 32")
    v = np.asarray(vals, dtype=np.int64)
    if v.size and (v.min() < 0 or v.max() > max_q(bits)):
        raise ValueError("field value out of range")
    v = v.astype(np.uint64)
    out = np.zeros((L * bits // 32, C), dtype=np.uint64)
    for i in range(L):
        word, off = divmod(i * bits, 32)
        out[word] |= (v[i] << np.uint64(off)) & _U32
        if off + bits > 32:           # the field straddles into the next word
            out[word + 1] |= v[i] >> np.uint64(32 - off)
    return out.astype(np.uint32).view(np.int32)


def unpack_fields(words: np.ndarray, bits: int, L: int) -> np.ndarray:
    """Inverse of pack_fields: int32 words [L*b/32, C] -> fields int64 [L, C].
    Uses logical shifts on the unsigned reinterpretation of each word."""
    u = np.ascontiguousarray(words).view(np.uint32).astype(np.uint64)
    if u.shape[0] * 32 != L * bits:
        raise ValueError("word count does not match L * bits / 32")
    mask = np.uint64(max_q(bits))
    out = np.empty((L, u.shape[1]), dtype=np.int64)
    for i in range(L):
        word, off = divmod(i * bits, 32)
        val = u[word] >> np.uint64(off)
        if off + bits > 32:
            val = val | (u[word + 1] << np.uint64(32 - off))
        out[i] = (val & mask).astype(np.int64)
    return out


def pack_along_k(q: np.ndarray, bits: int) -> np.ndarray:
    """qweight [K*b/32, N]: each column's K values packed along K."""
    return pack_fields(q, bits)


def pack_along_n(stored: np.ndarray, bits: int) -> np.ndarray:
    """qzeros [G, N*b/32]: each group row's N values packed along N."""
    return np.ascontiguousarray(pack_fields(np.asarray(stored).T, bits).T)


def unpack_along_k(qweight: np.ndarray, bits: int, K: int) -> np.ndarray:
    return unpack_fields(qweight, bits, K)


def unpack_along_n(qzeros: np.ndarray, bits: int, N: int) -> np.ndarray:
    return np.ascontiguousarray(unpack_fields(np.ascontiguousarray(np.asarray(qzeros).T), bits, N).T)


def convert_zeros_packed(qzeros: np.ndarray, bits: int, N: int, to_v2: bool):
    """Packed qzeros [G, N*b/32] in one format -> the other [P1-V2], plus the
    number of fields the target cannot hold exactly (v1 fields of 2^b - 1,
    saturated; v2 zeros of 0, stored as 0 = run-time zero 1)."""
    stored = unpack_along_n(qzeros, bits, N)
    if to_v2:
        lossy = int(np.count_nonzero(stored == max_q(bits)))
        conv = convert_zeros_v1_to_v2(stored, bits, saturate=True)
    else:
        lossy = int(np.count_nonzero(stored == 0))
        conv = convert_zeros_v2_to_v1(stored, bits)
    return pack_along_n(conv, bits), lossy


TILE_COLS = 16   # columns of one tile of the tiled qweight layout


# 4-bit words of the tiled layout hold their eight fields in pair order:
# nibble i holds the field that nibble PAIR_NIBBLES[i] holds in the checkpoint
# word, i.e. field 2i in nibble i and field 2i+1 in nibble i+4 (i < 4).
PAIR_NIBBLES = (0, 2, 4, 6, 1, 3, 5, 7)


def _permute_nibbles(w: np.ndarray, to_pairs: bool) -> np.ndarray:
    u = np.asarray(w).view(np.uint32)
    out = np.zeros_like(u)
    for i, src in enumerate(PAIR_NIBBLES):
        if to_pairs:
            out |= ((u >> np.uint32(4 * src)) & np.uint32(0xF)) << np.uint32(4 * i)
        else:
            out |= ((u >> np.uint32(4 * i)) & np.uint32(0xF)) << np.uint32(4 * src)
    return out.view(np.int32)


def repack_tiled(qweight: np.ndarray, bits: int) -> np.ndarray:
    """Checkpoint qweight [K*b/32, N] -> the tiled layout, int32 [N/16, K/32, b, 16].

    Word (t, c, r, j) is packed row c*b + r of column 16*t + j: each 16-column
    tile holds, chunk after chunk (32 rows of K), the b packed rows of that
    chunk, 16 words each.  For 2, 3 and 8 bits the bits inside a word are
    untouched; a 4-bit word holds its eight fields in pair order
    (PAIR_NIBBLES), so that each 16-bit half masked at one position gives two
    consecutive fields.  (An offline re-layout in the spirit of the page
    "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel", section
    6.1; the concrete order is this library's own, so the pages fix no
    expected value.)"""
    w = np.ascontiguousarray(qweight)
    R, N = w.shape
    if R % bits != 0 or N % TILE_COLS != 0:
        raise ValueError("qweight must be [K*b/32, N] with N % 16 == 0")
    C = R // bits
    t = np.ascontiguousarray(w.reshape(C, bits, N // TILE_COLS, TILE_COLS).transpose(2, 0, 1, 3))
    return _permute_nibbles(t, True) if bits == 4 else t


def unrepack_tiled(tiled: np.ndarray, bits: int, K: int, N: int) -> np.ndarray:
    """Inverse of repack_tiled: the tiled layout -> checkpoint qweight [K*b/32, N]."""
    t = np.asarray(tiled).reshape(N // TILE_COLS, K // 32, bits, TILE_COLS)
    if bits == 4:
        t = _permute_nibbles(np.ascontiguousarray(t), False)
    return np.ascontiguousarray(t.transpose(1, 2, 0, 3).reshape(K // 32 * bits, N))


def dequant_ref(qweight: np.ndarray, qzeros: np.ndarray, scales: np.ndarray,
                g_idx: Optional[np.ndarray], bits: int, group_size: int, is_v2: bool,
                K: int, N: int, cols: Optional[np.ndarray] = None, act: str = "fp16") -> np.ndarray:
    """W^[k, n] = fp16_rne((q[k,n] - z[g(k), n]) * s[g(k), n]) from packed data only.

    z = stored zero + zero_offset, zero_offset = 0 for v2 and 1 for v1
    [P1-ADJ]; the sum is a plain integer (a stored 2^b - 1 under v1 gives 2^b).
    ``cols`` optionally restricts the result to a subset of output columns.

    act="bf16": the layer of a bfloat16 model -- scales are bfloat16 values
    (given as floats, each exactly representable) and W^ is the product
    rounded once to bfloat16 (returned as float64 values); the pages name
    bfloat16 next to fp16 as the activation type (P3 section 1.2)."""
    if act not in ("fp16", "bf16"):
        raise ValueError("act must be 'fp16' or 'bf16'")
    G = num_groups(K, group_size)
    if cols is None:
        cols = np.arange(N)
    cols = np.asarray(cols, dtype=np.int64)
    q = unpack_along_k(np.ascontiguousarray(np.asarray(qweight)[:, cols]), bits, K)
    stored = unpack_along_n(qzeros, bits, N)[:, cols]
    zero_offset = 0 if is_v2 else 1
    z = stored + zero_offset
    g = group_of_rows(K, group_size, g_idx)
    if g.size and (g.min() < 0 or g.max() >= G):
        raise ValueError("g_idx entries must lie in [0, G)")
    if act == "bf16":
        s = np.asarray(scales, dtype=np.float64)[:, cols]
        if not np.array_equal(bf16_rne(s), s):
            raise ValueError("bf16 scales must be exact bfloat16 values")
        prod = (q - z[g]).astype(np.float64) * s[g]  # exact: <= 9 + 8 significant bits
        return bf16_rne(prod)
    s = np.asarray(scales, dtype=np.float16)[:, cols].astype(np.float64)
    prod = (q - z[g]).astype(np.float64) * s[g]     # exact: <= 9 + 11 significant bits
    return fp16_rne(prod)


def gemm_ref(x: np.ndarray, W_hat: np.ndarray) -> np.ndarray:
    """y = x @ W^ with both operands widened to fp64 (products are exact)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W_hat, dtype=np.float64)


def gptq_gemm_ref(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, K, N,
                  cols=None, act: str = "fp16") -> np.ndarray:
    """The whole path on the CPU: dequantize from the packed arrays, then multiply.
    act="bf16": x and scales hold bfloat16 values (see dequant_ref)."""
    return gemm_ref(x, dequant_ref(qweight, qzeros, scales, g_idx, bits, group_size,
                                   is_v2, K, N, cols=cols, act=act))


def sort_act_order(qweight: np.ndarray, g_idx: np.ndarray, bits: int, group_size: int, K: int):
    """Rows of an act-order layer sorted by group: perm = the stable order of
    g_idx, packed row fields q_sorted[i, n] = q[perm[i], n].  When every group
    has exactly group_size rows, row i of the sorted layer lies in group
    i // group_size, so the layer is an ordinary grouped one for x[:, perm]:
    sum_k x[m, k] W^[k, n] = sum_i x[m, perm[i]] W^[perm[i], n].  (Act order
    assigns rows to groups out of order: page "GPTQ quantization principles
    and engineering practice", section 3.4, desc_act; the row sort with a
    gathered x is this library's reading of how to run such a layer.)
    Returns (qweight_sorted [K*b/32, N], perm int32 [K])."""
    g = group_of_rows(K, group_size, g_idx)
    perm = np.argsort(g, kind="stable")
    if not np.array_equal(g[perm], np.arange(K) // group_size):
        raise ValueError("act-order groups are not all of group_size rows")
    q = unpack_along_k(qweight, bits, K)
    return pack_along_k(q[perm], bits), perm.astype(np.int32)


def moe_gemm_ref(x, experts, offsets, bits, group_size, is_v2, K, N, cols=None) -> np.ndarray:
    """Grouped GEMM over routed tokens: rows [offsets[e], offsets[e+1]) of x use
    expert e's packed weights; each expert's rows go through gptq_gemm_ref.
    `experts` is a list of (qweight, qzeros, scales, g_idx).  Rows of no expert
    are NaN (the GPU leaves them untouched).  (MoE models quantize their
    expert weights like dense layers: page "Weight-only INT4 quantization:
    GPTQ, AWQ and the Marlin kernel", section 7.)"""
    x = np.asarray(x)
    ncols = N if cols is None else len(cols)
    y = np.full((x.shape[0], ncols), np.nan)
    for e, (qw, qz, sc, gi) in enumerate(experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            y[r0:r1] = gptq_gemm_ref(x[r0:r1], qw, qz, sc, gi, bits, group_size, is_v2, K, N, cols=cols)
    return y


@dataclass
class QuantizedLayer:
    qweight: np.ndarray   # int32 [K*b/32, N]
    qzeros: np.ndarray    # int32 [G, N*b/32]
    scales: np.ndarray    # fp16 [G, N]
    g_idx: Optional[np.ndarray]
    bits: int
    group_size: int
    is_v2: bool
    q: np.ndarray         # int64 [K, N] unpacked codes
    zero: np.ndarray      # int64 [G, N] true zero points


def quantize_layer(W: np.ndarray, bits: int, group_size: int, sym: bool, is_v2: bool,
                   g_idx: Optional[np.ndarray] = None) -> QuantizedLayer:
    """Quantize, store zeros in the requested format, and pack."""
    q, zero, scale = quantize_minmax(W, bits, group_size, sym, g_idx)
    stored = store_zeros(zero, bits, is_v2)
    return QuantizedLayer(
        qweight=pack_along_k(q, bits),
        qzeros=pack_along_n(stored, bits),
        scales=scale,
        g_idx=None if g_idx is None else np.asarray(g_idx, dtype=np.int32),
        bits=bits, group_size=group_size, is_v2=is_v2, q=q, zero=zero)
