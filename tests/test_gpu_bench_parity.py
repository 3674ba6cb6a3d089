"""GPU parity for exactly the calls bench.py times (workload.BENCH_CASES).

Every benchmarked (workload, layer, M, qweight layout, activation type, entry
point) runs here through the same binding call and the same automatic kernel
choice as in the benchmark, so each kernel instantiation and launch shape the
benchmark reports has its result checked against the fp64 oracle:

- decode calls (M <= 16): every output column, max|y - y_ref| <= 5e-3 rms(y_ref)
  (bfloat16: plus the output's own rounding, 2^-8 |y_ref|);
- prefill calls (M > 16: the small-batch calls at 17-512 rows, M = 2048): at
  least 96 sampled columns (the oracle's fp64 product over the whole 2048 x K
  x N layer would take minutes on the host), spread so that every 256-column
  block tile of the kernel contributes.

Layers are quantized and packed by the oracle (seeded draws), the tiled layout
is the oracle's re-layout; nothing the GPU computes is fed back to the oracle.
"""
import numpy as np
import pytest

import oracle
import weight_only_bit_gptq_amd as gq
from workload import BENCH_CASES, WORKLOADS, draw_workload_layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 5e-3
OUT_ROUND_BF16 = 2.0 ** -8


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.library()
    return torch.device("cuda:0")


_layers = {}


def oracle_layer(wname, lname, M):
    """(draw, quantized layer) of a workload layer; cached per (workload, layer)
    with x drawn for the largest M the workload uses (x[:M] is the draw at M)."""
    key = (wname, lname)
    if key not in _layers:
        _layers.clear()
        wl = WORKLOADS[wname]
        layer = next(l for l in wl.layers if l.name == lname)
        d = draw_workload_layer(wl, layer, max(wl.Ms), seed=0)
        L = oracle.quantize_layer(d.W, wl.bits, wl.group_size, wl.sym, wl.is_v2, d.g_idx)
        d.W = None
        _layers[key] = (d, L)
    return _layers[key]


def sample_cols(N):
    """One random column in every 256-column block (the prefill kernel's block
    tile width), plus random columns up to 96 in all, plus the first and last."""
    rng = np.random.default_rng(N)
    blocks = np.arange(0, N, 256)
    cols = set((blocks + rng.integers(0, 256, size=blocks.size)).tolist()) | {0, N - 1}
    while len(cols) < 96:
        cols.add(int(rng.integers(0, N)))
    return np.array(sorted(c for c in cols if c < N))


def bf16_values(a):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(torch.bfloat16)
    return t, t.to(torch.float64).numpy()


@pytest.mark.parametrize("case", BENCH_CASES, ids=[c.key for c in BENCH_CASES])
def test_bench_case(dev, case):
    wl = WORKLOADS[case.workload]
    layer = next(l for l in wl.layers if l.name == case.layer)
    K, N, M = layer.K, layer.N, case.M
    d, L = oracle_layer(case.workload, case.layer, M)
    x = d.x[:M]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    qz = t(L.qzeros)
    if case.act == "bf16":
        sc_t, sc_ref = bf16_values(L.scales.astype(np.float32))
        x_t, x_ref = bf16_values(x.astype(np.float32))
        sc, xt = sc_t.to(dev), x_t.to(dev)
    else:
        sc, xt, sc_ref, x_ref = t(L.scales), t(x), L.scales, x
    gi = None if L.g_idx is None else t(L.g_idx)
    if case.entry == "gemm_sorted":
        qs, perm = oracle.sort_act_order(L.qweight, L.g_idx, wl.bits, wl.group_size, K)
        qw = t(oracle.repack_tiled(qs, wl.bits) if case.layout == "tiled" else qs)
        desc = gq.describe(xt, qw, qz, sc, None, wl.bits, wl.group_size, wl.is_v2)
        y = gq.gemm_sorted(xt, qw, qz, sc, t(perm), wl.bits, wl.group_size, wl.is_v2)
    else:
        qw = t(oracle.repack_tiled(L.qweight, wl.bits) if case.layout == "tiled" else L.qweight)
        desc = gq.describe(xt, qw, qz, sc, gi, wl.bits, wl.group_size, wl.is_v2)
        y = gq.gemm(xt, qw, qz, sc, gi, wl.bits, wl.group_size, wl.is_v2)
    cols = None if M <= 16 else sample_cols(N)
    ref = oracle.gptq_gemm_ref(x_ref, L.qweight, L.qzeros, sc_ref, L.g_idx, wl.bits, wl.group_size, wl.is_v2, K, N,
                               cols=cols, act=case.act)
    if cols is not None:
        y = y[:, torch.from_numpy(cols).to(dev)]
    yv = y.to(torch.float64).cpu().numpy()
    assert np.isfinite(yv).all(), desc
    rms = np.sqrt(np.mean(ref ** 2))
    bound = TOL * rms + (OUT_ROUND_BF16 * np.abs(ref) if case.act == "bf16" else 0.0)
    excess = np.abs(yv - ref) - bound
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[i] <= 0, f"{desc}: |y - y_ref| = {abs(yv[i] - ref[i]):.3e} at {i}, bound {np.broadcast_to(bound, ref.shape)[i]:.3e}"
