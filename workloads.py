"""Seeded synthetic inputs shaped like the linear layers the method serves.

This module only draws random numbers and names shapes; it holds none of the
quantization or GEMM arithmetic, so both the oracle side and the GPU side can
take their inputs from it without sharing any of the method's code.

Recipe (per workload shape, a fresh PCG64 stream seeded with 0):
  1. W = 0.02 * standard_normal((N, K)) in float32 (Linear layout, row = output channel);
  2. X = standard_normal((M, K)) in float32;
  3. a fixed set of round(p * K) input channels, drawn without replacement, is
     multiplied by f in every row (activation outlier channels);
  4. X is rounded to float16 (round-to-nearest-even), the dtype a preceding
     layer hands over in serving.
W is drawn first, so every M of one shape sees the same weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128


@dataclass(frozen=True)
class Shape:
    name: str
    K: int
    N: int


@dataclass(frozen=True)
class Workload:
    key: str
    description: str
    Ms: tuple
    shapes: tuple
    outlier_frac: float = 0.02
    outlier_gain: float = 20.0
    group: int = GROUP
    seed: int = 0


WORKLOADS = {
    "tiny": Workload(
        "tiny", "tiny W4A8 GEMM (M=16, K=512, N=512)", (16,),
        (Shape("tiny", 512, 512),)),
    "decode": Workload(
        "decode", "decode-shaped memory-bound GEMM (K=N=4096)", (1, 8, 32, 64),
        (Shape("square", 4096, 4096),)),
    "llama3_8b": Workload(
        "llama3_8b", "Llama-3-8B-shaped layer set at M=256", (256,),
        (Shape("qkv", 4096, 6144), Shape("o", 4096, 4096),
         Shape("gate_up", 4096, 28672), Shape("down", 14336, 4096))),
    "prefill": Workload(
        "prefill", "prefill compute-bound GEMM (M=4096, K=4096, N=14336)", (4096,),
        (Shape("prefill", 4096, 14336),), outlier_frac=0.01, outlier_gain=50.0),
    "qwen15_72b": Workload(
        "qwen15_72b", "Qwen1.5-72B-shaped layers", (64, 1024),
        (Shape("gate_up", 8192, 49152), Shape("down", 24576, 8192),
         Shape("qkv", 8192, 24576))),
}
ORDER = ("tiny", "decode", "llama3_8b", "prefill", "qwen15_72b")


def make_weights(N, K, seed=0):
    """W float32 [N, K] ~ 0.02 * N(0, 1)."""
    rng = np.random.default_rng(seed)
    return _weights(rng, N, K), rng


def _weights(rng, N, K):
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(0.02)
    return w


def make_activations(rng, M, K, outlier_frac, outlier_gain):
    """X float16 [M, K] ~ N(0, 1) with round(p*K) outlier channels scaled by f."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    idx = rng.choice(K, n_out, replace=False) if n_out else np.zeros(0, np.int64)
    x[:, idx] *= np.float32(outlier_gain)
    return x.astype(np.float16), idx


def make_case(workload: Workload, shape: Shape, M: int):
    """(W fp32 [N,K], X fp16 [M,K], outlier channel indices) for one case."""
    rng = np.random.default_rng(workload.seed)
    W = _weights(rng, shape.N, shape.K)
    X, idx = make_activations(rng, M, shape.K, workload.outlier_frac, workload.outlier_gain)
    return W, X, idx


def make_inputs(M, K, N, seed=0, outlier_frac=0.02, outlier_gain=20.0):
    """Ad-hoc case of any size with the same distributions."""
    rng = np.random.default_rng(seed)
    W = _weights(rng, N, K)
    X, idx = make_activations(rng, M, K, outlier_frac, outlier_gain)
    return W, X, idx


def algorithmic_bytes(M, K, N, group=GROUP):
    """HBM bytes the method must move for one GEMM (nibbles, group scale and
    zero at 1.5 B, fp16 channel scale, int8 activations, fp32 token scale,
    fp16 output)."""
    return (N * K // 2 + (N * K // group) * 3 // 2 + 2 * N + M * K + 4 * M + 2 * M * N)


def algorithmic_ops(M, K, N):
    return 2 * M * N * K
