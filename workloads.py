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


# ---------------------------------------------------------------------------
# decode attention over a 4-bit KV cache
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class AttnWorkload:
    key: str
    description: str
    B: int            # sequences (one new query token each)
    H: int            # query heads
    H_kv: int         # key/value heads
    D: int            # head dim
    len_lo: int       # context lengths drawn uniformly in [len_lo, len_hi]
    len_hi: int
    key_outlier_frac: float = 0.02
    key_outlier_gain: float = 10.0
    seed: int = 0


ATTN_WORKLOADS = {
    "llama3_8b_attn": AttnWorkload(
        "llama3_8b_attn", "Llama-3-8B decode attention (32 query / 8 KV heads, D=128), "
        "64 sequences of 512-2048 tokens", 64, 32, 8, 128, 512, 2048),
    "qwen15_72b_attn": AttnWorkload(
        "qwen15_72b_attn", "Qwen1.5-72B decode attention (64 heads, D=128), "
        "16 sequences of 512-2048 tokens", 16, 64, 64, 128, 512, 2048),
    "llama3_8b_long": AttnWorkload(
        "llama3_8b_long", "Llama-3-8B decode attention, 4 sequences of 8192-16384 tokens",
        4, 32, 8, 128, 8192, 16384),
}


def make_attention(B, H, H_kv, D, lens, seed=0, key_outlier_frac=0.02, key_outlier_gain=10.0):
    """(q [B,H,D], k [B,T,H_kv,D], v [B,T,H_kv,D]) float16 with T = max(lens):
    N(0, 1) values; per KV head a fixed set of round(p*D) key channels scaled
    by f (the key outlier channels smoothing targets). Draw order: the
    outlier channels of every head, then k, v, q."""
    rng = np.random.default_rng(seed)
    T = int(max(lens)) if len(lens) else 0
    n_out = int(round(key_outlier_frac * D))
    idx = [rng.choice(D, n_out, replace=False) for _ in range(H_kv)]
    k = rng.standard_normal((B, T, H_kv, D), dtype=np.float32)
    for h in range(H_kv):
        k[:, :, h, idx[h]] *= np.float32(key_outlier_gain)
    k = k.astype(np.float16)
    v = rng.standard_normal((B, T, H_kv, D), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((B, H, D), dtype=np.float32).astype(np.float16)
    return q, k, v


def attention_lens(w: AttnWorkload):
    """Context lengths [B] int32, uniform in [len_lo, len_hi] (own stream)."""
    rng = np.random.default_rng(w.seed + 1)
    return rng.integers(w.len_lo, w.len_hi + 1, size=w.B).astype(np.int32)


def make_attention_case(w: AttnWorkload):
    lens = attention_lens(w)
    q, k, v = make_attention(w.B, w.H, w.H_kv, w.D, lens, w.seed, w.key_outlier_frac,
                             w.key_outlier_gain)
    return q, k, v, lens


def attention_bytes(lens, H, H_kv, D):
    """HBM bytes one decode-attention call must move: per cached token and
    KV head the 4-bit key and value codes (D/2 bytes each) with an fp16 scale
    and a 4-bit zero apiece; the fp16 queries, outputs and smoothing factors."""
    tokens = int(np.sum(lens))
    B = len(lens)
    return tokens * H_kv * (D + 5) + 2 * B * H * D * 2 + 2 * H_kv * D


def algorithmic_bytes(M, K, N, group=GROUP):
    """HBM bytes the method must move for one GEMM (nibbles, group scale and
    zero at 1.5 B, fp16 channel scale, int8 activations, fp32 token scale,
    fp16 output)."""
    return (N * K // 2 + (N * K // group) * 3 // 2 + 2 * N + M * K + 4 * M + 2 * M * N)


def algorithmic_ops(M, K, N):
    return 2 * M * N * K
