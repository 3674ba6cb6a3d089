"""Seeded synthetic inputs for the GPTQ weight-only GEMM.

This module draws random numbers and nothing else: full-precision weights,
an outlier mask, an act-order group assignment and fp16 activations.  It holds
none of the method's arithmetic (no quantization, packing, dequantization or
contraction), so the CPU oracle and the HIP library can both consume what it
returns without sharing any computation.

Sources for the shapes and distributions:
- "Enhancing vLLM's support for the GPTQv2 format" (xxxxyu blog), section
  "Weight quantization of LLMs": b-bit integer weights with per-group
  scale/zero; section "From GPTQv1 to GPTQv2": the two zero-point formats.
- "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel"
  (aiinfraguide 4.3), section 1.1: decode reads every weight once per token,
  prefill is a dense contraction.
- "GPTQ principle and engineering practice" (rkmt.cn), section 3.5: roughly
  0.5% of entries are outliers; used only as the outlier rate of the 2-bit
  workload.

Draw order for one layer (one ``numpy.random.default_rng(seed)`` stream):
W, then the outlier mask (if any), then the act-order permutation (if any),
then x.  Because W is drawn first, a layer's weights do not depend on M.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


@dataclass(frozen=True)
class Layer:
    """One linear layer: x[M,K] @ W[K,N]."""
    name: str
    K: int
    N: int


@dataclass(frozen=True)
class Workload:
    """A named workload: layer shapes, batch sizes and the quantization recipe."""
    name: str
    layers: List[Layer]
    Ms: List[int]
    bits: int
    group_size: int
    sym: bool
    is_v2: bool
    sigma: float
    outlier_rate: float = 0.0
    outlier_mult: float = 10.0
    act_order: bool = False
    description: str = ""


# The workloads.  Shapes stand in for Llama-7B, Llama/Qwen and a 70B MLP;
# no trained weights are used anywhere.
WORKLOADS: Dict[str, Workload] = {
    "smoke_256": Workload(
        name="smoke_256",
        layers=[Layer("fc", 256, 256)],
        Ms=[1], bits=4, group_size=64, sym=False, is_v2=True, sigma=0.02,
        description="single 256x256 layer, 4-bit g64 asymmetric GPTQv2, M=1"),
    "llama7b_decode_w4g128": Workload(
        name="llama7b_decode_w4g128",
        layers=[Layer("qkv", 4096, 12288), Layer("o_proj", 4096, 4096),
                Layer("gate_up", 4096, 22016), Layer("down", 11008, 4096)],
        Ms=[1], bits=4, group_size=128, sym=True, is_v2=False, sigma=0.02,
        description="Llama-7B decode GEMVs, 4-bit g128 symmetric GPTQv1, M=1"),
    "llama7b_batch_w4g128": Workload(
        name="llama7b_batch_w4g128",
        layers=[Layer("qkv", 4096, 12288), Layer("o_proj", 4096, 4096),
                Layer("gate_up", 4096, 22016), Layer("down", 11008, 4096)],
        Ms=[17, 64, 128, 512], bits=4, group_size=128, sym=True, is_v2=False, sigma=0.02,
        description="the Llama-7B layers at small batches (M = 17-512: batched decode, short "
                    "prompts), 4-bit g128 symmetric GPTQv1"),
    "lowbit_decode_w2g64": Workload(
        name="lowbit_decode_w2g64",
        layers=[Layer("up", 4096, 12288), Layer("down", 12288, 4096)],
        Ms=[1, 4, 16], bits=2, group_size=64, sym=False, is_v2=True, sigma=0.02,
        outlier_rate=0.005, outlier_mult=10.0,
        description="2-bit g64 asymmetric GPTQv2 with 0.5% x10 outliers, M in {1,4,16}"),
    "actorder_decode_w3g128": Workload(
        name="actorder_decode_w3g128",
        layers=[Layer("up", 5120, 13824), Layer("down", 13824, 5120)],
        Ms=[16], bits=3, group_size=128, sym=False, is_v2=True, sigma=0.02,
        act_order=True,
        description="3-bit g128 asymmetric GPTQv2, act-order g_idx, M=16"),
    "mlp70b_prefill_w4g128": Workload(
        name="mlp70b_prefill_w4g128",
        layers=[Layer("up", 8192, 28672), Layer("down", 28672, 8192)],
        Ms=[2048], bits=4, group_size=128, sym=True, is_v2=False, sigma=0.015,
        description="70B MLP prefill, 4-bit g128 symmetric GPTQv1, M=2048"),
    "mlp70b_prefill_w8g128": Workload(
        name="mlp70b_prefill_w8g128",
        layers=[Layer("up", 8192, 28672), Layer("down", 28672, 8192)],
        Ms=[2048], bits=8, group_size=128, sym=False, is_v2=True, sigma=0.015,
        description="70B MLP prefill, 8-bit g128 asymmetric GPTQv2, M=2048"),
}



@dataclass(frozen=True)
class BenchCase:
    """One call the benchmark times: a workload layer at M rows, with qweight in
    the checkpoint layout or re-laid out into the tiled one, fp16 or bfloat16
    activations, through gptq_gemm (act-order layers: g_idx passed as is) or
    gptq_gemm_sorted (act-order rows sorted by group once at load).  The GPU
    parity tests run exactly these calls."""
    group: str                    # the bench line that reports it
    workload: str
    layer: str
    M: int
    layout: str                   # "tiled" | "checkpoint"
    act: str = "fp16"             # "fp16" | "bf16"
    entry: str = "gemm"           # "gemm" | "gemm_sorted"

    @property
    def key(self) -> str:
        return f"{self.group}:{self.workload}:{self.layer}:M{self.M}:{self.layout}:{self.act}:{self.entry}"


def _cases(group, wname, Ms, layout, act="fp16", entry="gemm"):
    wl = WORKLOADS[wname]
    return [BenchCase(group, wname, l.name, M, layout, act, entry) for l in wl.layers for M in Ms]


# Every GEMM call bench.py times, grouped by the line of its JSON output.
BENCH_CASES: List[BenchCase] = (
    _cases("decode", "llama7b_decode_w4g128", [1], "tiled")
    + _cases("decode_checkpoint", "llama7b_decode_w4g128", [1], "checkpoint")
    + _cases("decode_other", "lowbit_decode_w2g64", [1, 4, 16], "tiled")
    + _cases("decode_other", "actorder_decode_w3g128", [16], "tiled", entry="gemm_sorted")
    + _cases("decode_other", "actorder_decode_w3g128", [16], "checkpoint")
    + _cases("small_batch", "llama7b_batch_w4g128", [17, 64, 128, 512], "tiled")
    + _cases("prefill", "mlp70b_prefill_w4g128", [2048], "tiled")
    + _cases("prefill", "mlp70b_prefill_w8g128", [2048], "tiled")
    + _cases("prefill_checkpoint", "mlp70b_prefill_w4g128", [2048], "checkpoint")
    + _cases("bf16_decode", "llama7b_decode_w4g128", [1], "checkpoint", act="bf16")
    + _cases("bf16_decode_tiled", "llama7b_decode_w4g128", [1], "tiled", act="bf16")
    + _cases("bf16_prefill", "mlp70b_prefill_w4g128", [2048], "checkpoint", act="bf16")
    + _cases("bf16_prefill", "mlp70b_prefill_w4g128", [2048], "tiled", act="bf16")
)


def bench_cases(group: str) -> List[BenchCase]:
    return [c for c in BENCH_CASES if c.group == group]

@dataclass
class LayerDraw:
    """Random inputs for one layer."""
    W: np.ndarray                 # float32 [K, N]
    x: np.ndarray                 # float16 [M, K]
    g_idx: Optional[np.ndarray]   # int32 [K] or None
    outlier_mask: Optional[np.ndarray] = field(default=None, repr=False)


def draw_weights(rng: np.random.Generator, K: int, N: int, sigma: float,
                 outlier_rate: float = 0.0, outlier_mult: float = 10.0):
    """W ~ N(0, sigma^2) in float32; optionally a Bernoulli(outlier_rate) mask
    whose entries are multiplied by ``outlier_mult``."""
    W = rng.standard_normal((K, N), dtype=np.float32)
    W *= np.float32(sigma)
    mask = None
    if outlier_rate > 0.0:
        mask = rng.random((K, N)) < outlier_rate
        W[mask] *= np.float32(outlier_mult)
    return W, mask


def draw_act_order(rng: np.random.Generator, K: int, group_size: int) -> np.ndarray:
    """Act-order group assignment: a seeded permutation of the K rows, cut into
    consecutive runs of ``group_size``; row perm[i] belongs to group
    i // group_size, so every group has exactly ``group_size`` rows."""
    perm = rng.permutation(K)
    g_idx = np.empty(K, dtype=np.int32)
    g_idx[perm] = (np.arange(K) // group_size).astype(np.int32)
    return g_idx


def draw_activations(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """x ~ N(0, 1) drawn in float32 and rounded to float16."""
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def draw_layer(K: int, N: int, M: int, *, sigma: float, group_size: int,
               outlier_rate: float = 0.0, outlier_mult: float = 10.0,
               act_order: bool = False, seed: int = 0) -> LayerDraw:
    """All random inputs of one layer, in the fixed draw order."""
    rng = np.random.default_rng(seed)
    W, mask = draw_weights(rng, K, N, sigma, outlier_rate, outlier_mult)
    g_idx = draw_act_order(rng, K, group_size) if act_order else None
    x = draw_activations(rng, M, K)
    return LayerDraw(W=W, x=x, g_idx=g_idx, outlier_mask=mask)


def draw_workload_layer(wl: Workload, layer: Layer, M: int, seed: int = 0) -> LayerDraw:
    return draw_layer(layer.K, layer.N, M, sigma=wl.sigma, group_size=wl.group_size,
                      outlier_rate=wl.outlier_rate, outlier_mult=wl.outlier_mult,
                      act_order=wl.act_order, seed=seed)


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniformly random int32 words (every bit pattern equally likely); used by
    edge-case tests that need packed arrays whose fields cover the full range."""
    return rng.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.int32)
