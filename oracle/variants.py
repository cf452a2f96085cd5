"""Plain CPU oracle for the comparison GEMMs the pages set QoQ against.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
executes this module: only the tests and the benchmark's CPU-baseline leg
do. It shares no code with the HIP library.

The pages measure QoQ's W4A8 GEMM against other low-bit GEMM families
("QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
Serving", velog study notes, sections "문제 정의" and "Background"; the QServe
abstract): W8A8 with per-channel weights and per-token activations, whose
GEMM needs no dequantization at all; weight-only W4A16, whose 4-bit weights
are dequantized to fp16 for fp16 matrix units; and per-group W4A4, whose
INT32 partial sums must be converted and scaled inside the main loop for
every group. The
pages give no arithmetic for either; the readings below are the plainest
ones the rest supports (listed again in the design notes):

* W8A8: per-channel symmetric INT8 weights over the full range [-127, 127]
  with an fp16 scale s = fp16(fp32(absmax / 127)), codes
  clamp(rne(fp32(w / fp32(s))), -127, 127) -- the QoQ level-1 step with the
  whole INT8 range instead of the protective range; activations as QoQ's
  (per-token symmetric INT8); y = acc * s_x[m] * s[n].
* W4A16: per-group (128 inputs) asymmetric UINT4 weights with an fp16 scale
  and a UINT4 zero (the weight-only format the pages' W4A16 baselines serve):
  lo = min(0, min w), hi = max(0, max w), s = fp16(fp32(fp32(hi - lo) / 15)),
  z = clamp(rne(fp32(-lo / fp32(s))), 0, 15), q = clamp(rne(fp32(w /
  fp32(s))) + z, 0, 15) (all-zero group: s = 0, q = z = 0); dequantized to
  fp16 as w16 = fp16((q - z) * s); activations stay fp16; y = x @ w16^T.
* W4A4: per-group (128 inputs) symmetric INT4 in [-7, 7] for both operands:
  weights with an fp16 scale per (channel, group), s_w = fp16(fp32(a / 7)),
  codes clamp(rne(fp32(w / fp32(s_w))), -7, 7); activations with an fp32
  scale per (token, group), inv = fp32(7 / a), codes
  clamp(rne(fp32(x * inv)), -7, 7), s_a = fp32(a / 7); all-zero groups get
  scale 0 and codes 0. The GEMM forms the exact integer partial sum of each
  group and accumulates y = sum_g P[m, n, g] * s_a[m, g] * s_w[n, g] in
  floating point: the partial-sum dequantization the pages single out.

Floating-point steps that decide an integer are IEEE fp32 (correctly rounded
division, round half to even), as in the kernels; the rest is exact (int64)
or fp64. Pins: tests/variant_pins.py.
"""
from __future__ import annotations

import numpy as np

from .qoq_oracle import level1_per_channel, quantize_act, int_gemm, epilogue

W8_MAX = 127
INT4_MAX = 7


# --------------------------------------------------------------------------
# W8A8: per-channel INT8 weights, per-token INT8 activations
# --------------------------------------------------------------------------
def w8a8_quantize_weights(W):
    """Per-output-channel symmetric INT8 over [-127, 127], fp16 scale.

    The same definition as QoQ's level 1 with the full INT8 range as bound.
    Returns s float16 [N], q8 int16 [N, K].
    """
    return level1_per_channel(W, protect=W8_MAX)


def w8a8_linear(x, W):
    """Whole W8A8 path on the CPU: y = (x8 @ q8^T) * s_x * s."""
    s, q8 = w8a8_quantize_weights(W)
    x8, s_x = quantize_act(x)
    acc = int_gemm(x8, q8)
    return {"acc": acc, "y": epilogue(acc, s_x, s), "x8": x8, "s_x": s_x, "q8": q8, "s": s}


# --------------------------------------------------------------------------
# W4A4: per-group INT4 weights and activations, partial sums scaled per group
# --------------------------------------------------------------------------
def _grouped(a, group):
    rows, k = a.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    return a.reshape(rows, k // group, group)


def w4a4_quantize_weights(W, group=128):
    """Per-(channel, group) symmetric INT4 in [-7, 7] with an fp16 scale.

    Returns s_w float16 [N, K/group], q int8 [N, K].
    """
    W = np.asarray(W, dtype=np.float32)
    g = _grouped(W, group)
    absmax = np.max(np.abs(g), axis=2)                       # exact
    s_w = (absmax / np.float32(INT4_MAX)).astype(np.float16)  # fp32 division, RNE to fp16
    s_back = s_w.astype(np.float32)
    q = np.zeros(g.shape, dtype=np.int8)
    live = s_back != 0
    if np.any(live):
        ratio = g[live] / s_back[live][:, None]               # fp32 division
        q[live] = np.clip(np.rint(ratio), -INT4_MAX, INT4_MAX).astype(np.int8)
    return s_w, q.reshape(W.shape)


def w4a4_quantize_act(x, group=128):
    """Per-(token, group) symmetric INT4 in [-7, 7] with an fp32 scale.

    inv = fp32(7 / absmax), codes clamp(rne(fp32(x * inv)), -7, 7),
    s_a = fp32(absmax / 7). Returns q int8 [M, K], s_a float32 [M, K/group].
    """
    xf = np.asarray(x, dtype=np.float16).astype(np.float32)
    g = _grouped(xf, group)
    absmax = np.max(np.abs(g), axis=2)
    s_a = np.zeros(absmax.shape, dtype=np.float32)
    q = np.zeros(g.shape, dtype=np.int8)
    live = absmax != 0
    if np.any(live):
        inv = np.float32(INT4_MAX) / absmax[live]            # fp32 division
        prod = g[live] * inv[:, None]                        # fp32 product
        q[live] = np.clip(np.rint(prod), -INT4_MAX, INT4_MAX).astype(np.int8)
        s_a[live] = absmax[live] / np.float32(INT4_MAX)
    return q.reshape(xf.shape), s_a


def w4a4_partial_sums(xq, wq, group=128):
    """P[m, n, g] = sum over the inputs k of group g of xq[m, k] * wq[n, k]
    (int64, literal per-group products)."""
    a = _grouped(np.asarray(xq, dtype=np.int64), group)      # [M, G, group]
    b = _grouped(np.asarray(wq, dtype=np.int64), group)      # [N, G, group]
    return np.einsum("mgk,ngk->mng", a, b)


def w4a4_linear(x, W, group=128):
    """Whole W4A4 path: y = sum_g P[:, :, g] * s_a[:, g] * s_w[:, g] in fp64.

    Also returns `term_abs` = sum_g |P * s_a * s_w|, the scale of the
    rounding error any floating-point accumulation order can make.
    """
    s_w, wq = w4a4_quantize_weights(W, group)
    xq, s_a = w4a4_quantize_act(x, group)
    P = w4a4_partial_sums(xq, wq, group).astype(np.float64)
    scale = s_a.astype(np.float64)[:, None, :] * s_w.astype(np.float64)[None, :, :]
    terms = P * scale
    return {"y": terms.sum(axis=2), "term_abs": np.abs(terms).sum(axis=2), "P": P,
            "xq": xq, "s_a": s_a, "wq": wq, "s_w": s_w}


# --------------------------------------------------------------------------
# W4A16: per-group UINT4 weights dequantized to fp16, fp16 activations
# --------------------------------------------------------------------------
def w4a16_quantize_weights(W, group=128):
    """Per-(channel, group) asymmetric UINT4 with fp16 scale and UINT4 zero.

    Returns q uint8 [N, K] (0..15), s float16 [N, K/group], z uint8 [N, K/group].
    """
    W = np.asarray(W, dtype=np.float32)
    g = _grouped(W, group)
    lo = np.minimum(np.float32(0), g.min(axis=2))
    hi = np.maximum(np.float32(0), g.max(axis=2))
    s = ((hi - lo) / np.float32(15)).astype(np.float16)        # fp32 ops, RNE to fp16
    s_back = s.astype(np.float32)
    z = np.zeros(s.shape, dtype=np.int64)
    q = np.zeros(g.shape, dtype=np.int64)
    live = s_back != 0
    if np.any(live):
        z[live] = np.clip(np.rint(-lo[live] / s_back[live]), 0, 15).astype(np.int64)
        codes = np.rint(g[live] / s_back[live][:, None]).astype(np.int64)
        q[live] = np.clip(codes + z[live][:, None], 0, 15)
    return q.reshape(W.shape).astype(np.uint8), s, z.astype(np.uint8)


def w4a16_dequantize(q, s, z, group=128):
    """w16 = fp16((q - z) * s): the product of a small integer and an fp16
    value is exact in fp64, then rounded once to fp16."""
    q = _grouped(np.asarray(q, dtype=np.int64), group)
    prod = (q - np.asarray(z, dtype=np.int64)[:, :, None]) * \
        np.asarray(s, dtype=np.float16).astype(np.float64)[:, :, None]
    n_rows = q.shape[0]
    return prod.reshape(n_rows, -1).astype(np.float16)


def w4a16_linear(x, W, group=128):
    """Whole W4A16 path: y = x16 @ w16^T in fp64, with term_abs =
    |x16| @ |w16|^T (the scale of any accumulation order's rounding)."""
    q, s, z = w4a16_quantize_weights(W, group)
    w16 = w4a16_dequantize(q, s, z, group)
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    wf = w16.astype(np.float64)
    return {"y": xf @ wf.T, "term_abs": np.abs(xf) @ np.abs(wf).T, "q": q, "s": s, "z": z,
            "w16": w16}
