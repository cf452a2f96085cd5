"""Plain CPU oracle for the KV4 decode attention with SmoothAttention scaling.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
executes this module: only the tests and the benchmark's CPU-baseline leg
do. It shares no code with the HIP library.

What the pages fix ("QServe: W4A8KV4 Quantization and System Co-design for
Efficient LLM Serving", velog study notes, sections "Insight" and "Methods /
1) Algorithm: QoQ"; the QServe abstract; "Part5 LLM部署技术" section 3): the
key/value cache is held in 4 bits; SmoothAttention moves the quantization
difficulty of the keys onto the queries, which stay unquantized; the fused
attention over the 4-bit cache is memory-bound. The pages give no formula
for either, so the plainest readings the rest supports are taken (listed
again in the design notes):

* KV4 format: every cached vector of one token and one key/value head (the
  head_dim = 128 values) is one group of the per-group UINT4 format the
  pages' weight-only baselines use (the same reading as the W4A16 weights):
  lo = min(0, min x), hi = max(0, max x), s = fp16(fp32(fp32(hi - lo) / 15)),
  z = clamp(rne(fp32(-lo / fp32(s))), 0, 15), code = clamp(rne(fp32(x /
  fp32(s))) + z, 0, 15); an all-zero vector gets s = 0, codes and zero 0.
  The cached value it stands for is (code - z) * s.
* SmoothAttention: the SmoothQuant migration ("Part5 LLM部署技术" section
  1.1: a per-channel factor from the calibration maxima with a migration
  strength) applied with the keys as the hard-to-quantize side and the
  queries, which are never quantized, taking the factor:
  lambda[h, d] = fp16(sqrt(fp32(max_t |K[t, h, d]|))) (strength 1/2; 1 for
  an all-zero channel). Keys are divided by lambda before quantization,
  k~ = fp32(k) / fp32(lambda); queries are multiplied by it,
  q~ = fp16(fp32(q) * fp32(lambda)). (q lambda) . (k / lambda) = q . k, so
  only the quantization error moves.
* Attention: one new query token per sequence (decode), query head h reads
  key/value head h // (H / H_kv) (grouped-query attention), scores
  q~ . k^ / sqrt(D) over the first len_b cached tokens, softmax, output the
  softmax-weighted sum of the v^ vectors; an empty context gives 0.

Floating-point steps that decide a stored value (lambda, s, z, codes, q~)
are IEEE fp32 with round half to even, as in the kernels; the attention
itself is evaluated in fp64. Pins: tests/kv4_pins.py.
"""
from __future__ import annotations

import numpy as np

from .variants import w4a16_quantize_weights


def smooth_factors(k_calib):
    """lambda [H_kv, D] fp16 from calibration keys [..., H_kv, D]:
    fp16(sqrt(fp32(max |k|))) per (head, channel), 1 where the max is 0."""
    k = np.asarray(k_calib, dtype=np.float16).astype(np.float32)
    h, d = k.shape[-2:]
    a = np.max(np.abs(k.reshape(-1, h, d)), axis=0)          # exact (fp16 values)
    lam = np.sqrt(a).astype(np.float16)                       # fp32 sqrt, RNE to fp16
    lam[a == 0] = np.float16(1.0)
    return lam


def kv4_quantize(x):
    """Per-vector UINT4 of x [..., D] (fp32): codes uint8 [..., D], s fp16
    [...], z uint8 [...] -- one group of the W4A16 format per vector."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    q, s, z = w4a16_quantize_weights(x.reshape(-1, d), group=d)
    return q.reshape(x.shape), s.reshape(x.shape[:-1]), z.reshape(x.shape[:-1])


def kv4_dequantize(codes, s, z):
    """(code - z) * s, exact in fp64."""
    c = np.asarray(codes, dtype=np.int64)
    zz = np.asarray(z, dtype=np.int64)[..., None]
    return (c - zz) * np.asarray(s, dtype=np.float16).astype(np.float64)[..., None]


def kv4_encode(k, v, lam):
    """Cache contents for keys and values [..., H_kv, D] (fp16): keys smoothed
    (divided by lambda in fp32) then quantized, values quantized as they are.
    Returns dict(kc, ks, kz, vc, vs, vz)."""
    kf = np.asarray(k, dtype=np.float16).astype(np.float32)
    vf = np.asarray(v, dtype=np.float16).astype(np.float32)
    ksm = kf / np.asarray(lam, dtype=np.float16).astype(np.float32)   # fp32 division
    kc, ks, kz = kv4_quantize(ksm)
    vc, vs, vz = kv4_quantize(vf)
    return dict(kc=kc, ks=ks, kz=kz, vc=vc, vs=vs, vz=vz)


def smooth_query(q, lam, group):
    """q~ [B, H, D] fp16 = fp16(fp32(q) * fp32(lambda of the head's KV head))."""
    qf = np.asarray(q, dtype=np.float16).astype(np.float32)
    lam_h = np.repeat(np.asarray(lam, dtype=np.float16).astype(np.float32), group, axis=0)
    return (qf * lam_h[None, :, :]).astype(np.float16)


def attention_core(qs, kh, vh, lens, group):
    """Decode attention in fp64 on given query vectors qs [B, H, D] and
    cached key / value vectors kh, vh [B, T, H_kv, D]: head h reads KV head
    h // group, tokens t < lens[b]. Returns (o [B, H, D], a [B, H, D],
    r [B, H]) with a = sum_t p_t |v_t| / sum_t p_t (the scale of any rounding
    of the weighted sum, per output) and r = max_t sum_d |q_d k_t,d| /
    sqrt(D) (the scale of any rounding of a score)."""
    qs = np.asarray(qs, dtype=np.float64)
    B, H, D = qs.shape
    o = np.zeros((B, H, D))
    a = np.zeros((B, H, D))
    r = np.zeros((B, H))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(H):
            hk = h // group
            k = kh[b, :n, hk, :]                              # [n, D]
            v = vh[b, :n, hk, :]
            q = qs[b, h]
            sc = (k @ q) / np.sqrt(D)
            w = np.exp(sc - sc.max())
            o[b, h] = (w @ v) / w.sum()
            a[b, h] = (w @ np.abs(v)) / w.sum()
            r[b, h] = float((np.abs(k) @ np.abs(q)).max() / np.sqrt(D))
    return o, a, r


def kv4_decode_attention(q, lam, enc, lens, group):
    """The whole path on the CPU: smoothed query, dequantized cache,
    attention. Returns dict(o, a, r, qs)."""
    qs = smooth_query(q, lam, group)
    kh = kv4_dequantize(enc["kc"], enc["ks"], enc["kz"])
    vh = kv4_dequantize(enc["vc"], enc["vs"], enc["vz"])
    o, a, r = attention_core(qs.astype(np.float64), kh, vh, lens, group)
    return dict(o=o, a=a, r=r, qs=qs)


def fp16_decode_attention(q, k, v, lens, group):
    """The comparison point: the same attention on an fp16 cache, queries
    unsmoothed (smoothing changes nothing without quantization). Returns
    dict(o, a, r)."""
    o, a, r = attention_core(np.asarray(q, dtype=np.float16).astype(np.float64),
                             np.asarray(k, dtype=np.float16).astype(np.float64),
                             np.asarray(v, dtype=np.float16).astype(np.float64), lens, group)
    return dict(o=o, a=a, r=r)
