"""gptq_gemm_noalloc (the entry point that allocates nothing) against gptq_gemm.

Called through the C ABI via the binding: two calls in a row, the second with
a smaller input, must give gptq_gemm's result bit for bit (same launch plan,
same kernels, same split-K order) and the oracle's within the GEMM bar; so must
replays of a graph that captured it.
"""
import numpy as np
import pytest

import oracle
import weight_only_bit_gptq_amd as gq
from workload import draw_layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

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


def layer(K, N, M, bits, gs, seed, act=False):
    d = draw_layer(K, N, M, sigma=0.02, group_size=gs, act_order=act, seed=seed)
    L = oracle.quantize_layer(d.W, bits, gs, False, True, d.g_idx)
    return d, L


def upload(d, L, dev):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t(d.x), t(L.qweight), t(L.qzeros), t(L.scales), None if L.g_idx is None else t(L.g_idx)


def check(y, d, L, K, N, bits, gs, what):
    ref = oracle.gptq_gemm_ref(d.x, L.qweight, L.qzeros, L.scales, L.g_idx, bits, gs, True, K, N)
    yv = y.float().cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.isfinite(yv).all(), what
    assert np.max(np.abs(yv - ref)) <= TOL * rms, what


# (K, N, M, bits, group size, act order): two split-K decode shapes, the second
# smaller, then an unsplit decode, an act-order decode and a prefill shape
CALLS = [(8192, 1024, 4, 4, 128, False), (8192, 256, 1, 2, 64, False), (4096, 2048, 1, 4, 128, False),
         (4096, 512, 16, 3, 128, True), (1024, 256, 40, 8, 128, False)]


def test_noalloc_matches_gemm_two_calls(dev):
    for i, (K, N, M, bits, gs, act) in enumerate(CALLS):
        d, L = layer(K, N, M, bits, gs, seed=100 + i, act=act)
        x, qw, qz, sc, gi = upload(d, L, dev)
        desc = gq.describe(x, qw, qz, sc, gi, bits, gs, True)
        if i < 2:
            assert k_splits(desc) > 1, desc
        want = gq.gemm(x, qw, qz, sc, gi, bits, gs, True)
        out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        got = gq.gemm_noalloc(x, qw, qz, sc, gi, bits, gs, True, out=out)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (i, desc)
        check(got, d, L, K, N, bits, gs, f"call {i}: {desc}")


def test_noalloc_prefill_split_within_scratch(dev):
    """A prefill shape whose split-K partial sums fit gptq_gemm's workspace
    but not the 2 MiB scratch: the no-allocation call splits K less (here not
    at all), so it matches the oracle to the GEMM bar and gptq_gemm to the
    rounding of the fp32 sums' order; called twice, the second time smaller."""
    for i, (K, N, M) in enumerate(((4096, 12288, 64), (4096, 1024, 80))):
        d, L = layer(K, N, M, 4, 128, seed=300 + i)
        x, qw, qz, sc, gi = upload(d, L, dev)
        desc = gq.describe(x, qw, qz, sc, gi, 4, 128, True)
        assert desc.startswith(("gptq::prefill_kernel", "gptq::prefill_small_kernel")), desc
        assert k_splits(desc) > 1, desc
        want = gq.gemm(x, qw, qz, sc, gi, 4, 128, True)
        out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        got = gq.gemm_noalloc(x, qw, qz, sc, gi, 4, 128, True, out=out)
        torch.cuda.synchronize()
        check(got, d, L, K, N, 4, 128, f"call {i}: {desc}")
        diff = (got.float() - want.float()).abs().max().item()
        assert diff <= TOL * want.float().pow(2).mean().sqrt().item(), (i, diff)


def test_noalloc_graph_replays(dev):
    """Captured (no allocation can happen under capture), replayed three times
    with eager work in between: every replay equals the eager result."""
    K, N, M, bits, gs = 8192, 512, 2, 4, 128
    d, L = layer(K, N, M, bits, gs, seed=200)
    x, qw, qz, sc, gi = upload(d, L, dev)
    want = gq.gemm(x, qw, qz, sc, gi, bits, gs, True)
    out = torch.zeros((M, N), dtype=torch.float16, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gq.gemm_noalloc(x, qw, qz, sc, gi, bits, gs, True, out=out)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gq.gemm_noalloc(x, qw, qz, sc, gi, bits, gs, True, out=out)
    # a smaller eager call between replays reuses the same scratch
    d2, L2 = layer(8192, 256, 1, 2, 64, seed=201)
    x2, qw2, qz2, sc2, _ = upload(d2, L2, dev)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
        o2 = torch.empty((1, 256), dtype=torch.float16, device=dev)
        gq.gemm_noalloc(x2, qw2, qz2, sc2, None, 2, 64, True, out=o2)
        torch.cuda.synchronize()
        check(o2, d2, L2, 8192, 256, 2, 64, f"eager call after replay {rep}")
