"""Plain CPU oracle for the QoQ W4A8 GEMM with progressive group quantization.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
executes this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg do. It shares no code, tables or constants with the HIP
library; the only thing the two sides have in common is the seeded input
generator in ``workloads.py``, which holds none of the method's arithmetic.

Sources (the pages, cited by title and section):

* "QServe: Cuantificación W4A8KV4 y Co-diseño del Sistema ..." (abstract):
  W4A8KV4 = 4-bit weights, 8-bit activations; progressive quantization keeps
  the dequantization overhead of the W4A8 GEMM low; weight dequantization
  and partial-sum dequantization are the overheads being removed.
* "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
  Serving" (velog study notes):
    - "Background": W8A8 is per-channel weight + per-token activation (the
      granularity labels on that page are shifted by one item; see the
      readings below), per-group = own scale/zero per sub-channel group, and
      per-group W4A4 must dequantize INT32 partial sums inside the main loop.
    - "Methods / 1) Algorithm: QoQ": weights are first quantized to 8 bit
      with per-channel FP16 scales, then the 8-bit intermediates to 4 bit,
      so that every GEMM operation runs on INT8 matrix units.
    - "Methods / 2) System: QServe": the protective range of progressive
      quantization enables register-level-parallel INT4->INT8 dequantization
      in the order "subtraction after multiplication".
* "Part5 LLM部署技术", section 3 (QServe): fused kernels avoid dequantizing
  partial sums, so floating-point scales are applied once.

Readings where the pages are silent (each is also listed with its
justification in the design notes):

* protective range R = 119: level-1 codes lie in [-119, 119]; this is the
  largest R for which every level-2 dequantized weight stays inside INT8
  (checked exhaustively by the tests; R = 120 overflows);
* level 1 is symmetric, scale = fp16(fp32(absmax / 119)), codes
  clamp(rne(fp32(w / fp32(s1))), -119, 119), zero row -> scale 0, codes 0;
* level 2 is asymmetric per group of G inputs of one output channel:
  lo = min(0, min q8), hi = max(0, max q8), s2 = max(1, ceil((hi-lo)/15)),
  z = rne(-lo / s2), q4 = clamp(rne(q8 / s2) + z, 0, 15), all in exact
  integer arithmetic with round-half-to-even;
* dequantization: w8 = q4 * s2 - z * s2 (multiply first, then subtract the
  pre-multiplied zero);
* activations: symmetric per token, inv = fp32(127 / absmax),
  x8 = clamp(rne(fp32(x * inv)), -127, 127), s_x = fp32(absmax / 127);
  zero row -> s_x = 0, codes 0;
* epilogue: y = acc * s_x[m] * s1[n], computed here in fp64.

All floating-point steps that decide an integer are done in IEEE fp32 with
correctly rounded division and round-half-to-even, the precision the kernel
uses; everything downstream of the integer codes is exact (int64) or fp64.

Parity pins for every function are in tests/test_oracle.py; none of the
functions here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# Level-1 protective range (reading: see module docstring).
PROTECT = 119
# Activation code bound: symmetric INT8 without -128.
ACT_MAX = 127
# Level-2 code range: UINT4.
Q4_MAX = 15


# --------------------------------------------------------------------------
# exact integer helpers
# --------------------------------------------------------------------------
def rne_div(num, den):
    """Round-half-to-even of the exact rational num/den, den > 0 (int64)."""
    num = np.asarray(num, dtype=np.int64)
    den = np.asarray(den, dtype=np.int64)
    quo = np.floor_divide(num, den)
    rem = num - quo * den  # 0 <= rem < den
    twice = 2 * rem
    round_up = (twice > den) | ((twice == den) & (quo % 2 != 0))
    return quo + round_up.astype(np.int64)


def ceil_div(num, den):
    """Ceiling of num/den for den > 0 (int64)."""
    num = np.asarray(num, dtype=np.int64)
    den = np.asarray(den, dtype=np.int64)
    return -np.floor_divide(-num, den)


# --------------------------------------------------------------------------
# weights: progressive group quantization
# --------------------------------------------------------------------------
def level1_per_channel(W, protect=PROTECT):
    """Level 1: per-output-channel symmetric INT8 with an FP16 scale.

    Pages: velog notes, "Methods / 1) Algorithm: QoQ" (first to 8 bit with
    per-channel FP16 scales) and "Methods / 2) System: QServe" (the 8-bit
    intermediate is kept inside a protective range).

    W: float32 [N, K] in Linear layout (row n = output channel n).
    Returns s1 float16 [N], q8 int16 [N, K] with |q8| <= protect.
    """
    W = np.asarray(W, dtype=np.float32)
    absmax = np.max(np.abs(W), axis=1)                      # exact
    s1_f32 = absmax / np.float32(protect)                   # fp32, correctly rounded
    s1 = s1_f32.astype(np.float16)                          # RNE to fp16
    s1_back = s1.astype(np.float32)
    q8 = np.zeros(W.shape, dtype=np.int16)
    live = s1_back != 0
    if np.any(live):
        ratio = W[live] / s1_back[live][:, None]            # fp32 division
        codes = np.clip(np.rint(ratio), -protect, protect)  # RNE, then clamp
        q8[live] = codes.astype(np.int16)
    return s1, q8


def level2_per_group(q8, group):
    """Level 2: per-group asymmetric UINT4 with integer scale s2, UINT4 zero z.

    Pages: velog notes, "Methods / 1) Algorithm: QoQ" (the 8-bit
    intermediates are quantized again to 4 bit) and "Background" (per-group
    means each sub-channel group has its own scale and zero point).

    q8: integer [N, K], K % group == 0.
    Returns q4 uint8 [N, K] (0..15), s2 int16 [N, K/group] (1..16),
    z uint8 [N, K/group] (0..15).
    """
    q8 = np.asarray(q8, dtype=np.int64)
    n_rows, k = q8.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    grouped = q8.reshape(n_rows, k // group, group)
    lo = np.minimum(0, grouped.min(axis=2))
    hi = np.maximum(0, grouped.max(axis=2))
    s2 = np.maximum(1, ceil_div(hi - lo, Q4_MAX))
    z = rne_div(-lo, s2)
    q4 = np.clip(rne_div(grouped, s2[:, :, None]) + z[:, :, None], 0, Q4_MAX)
    return (q4.reshape(n_rows, k).astype(np.uint8),
            s2.astype(np.int16), z.astype(np.uint8))


def dequantize_level2(q4, s2, z, group):
    """INT8 weights from UINT4 codes: w8 = q4*s2 - (z*s2).

    Pages: velog notes, "Methods / 2) System: QServe" (subtraction after
    multiplication; the product z*s2 is a per-group constant).
    Returns int64 [N, K].
    """
    q4 = np.asarray(q4, dtype=np.int64)
    n_rows, k = q4.shape
    s2 = np.asarray(s2, dtype=np.int64)
    z = np.asarray(z, dtype=np.int64)
    scaled = q4.reshape(n_rows, k // group, group) * s2[:, :, None]
    zero_term = (z * s2)[:, :, None]
    return (scaled - zero_term).reshape(n_rows, k)


def quantize_weights(W, group=128, protect=PROTECT):
    """Progressive group quantization of W [N, K]: level 1 then level 2."""
    s1, q8 = level1_per_channel(W, protect)
    q4, s2, z = level2_per_group(q8, group)
    return {"s1": s1, "q8": q8, "q4": q4, "s2": s2, "z": z}


# --------------------------------------------------------------------------
# activations: per-token symmetric INT8
# --------------------------------------------------------------------------
def quantize_act(x):
    """Per-token (per-row) symmetric INT8 quantization of x fp16 [M, K].

    Pages: abstract (8-bit activations) and velog notes, "Background"
    (per-token activation quantization paired with per-channel weights).
    Returns x8 int8 [M, K], s_x float32 [M].
    """
    xf = np.asarray(x, dtype=np.float16).astype(np.float32)
    absmax = np.max(np.abs(xf), axis=1) if xf.shape[1] else np.zeros(xf.shape[0], np.float32)
    s_x = np.zeros(xf.shape[0], dtype=np.float32)
    x8 = np.zeros(xf.shape, dtype=np.int8)
    live = absmax != 0
    if np.any(live):
        inv = np.float32(ACT_MAX) / absmax[live]             # fp32 division
        prod = xf[live] * inv[:, None]                       # fp32 product
        x8[live] = np.clip(np.rint(prod), -ACT_MAX, ACT_MAX).astype(np.int8)
        s_x[live] = absmax[live] / np.float32(ACT_MAX)
    return x8, s_x


# --------------------------------------------------------------------------
# GEMM: exact integer accumulation, then one floating-point scaling
# --------------------------------------------------------------------------
def int_gemm(x8, w8):
    """acc[m, n] = sum_k x8[m, k] * w8[n, k] in int64 (literal definition).

    Pages: velog notes, "Methods / 1) Algorithm: QoQ" (all GEMM operations
    are INT8 x INT8) and "Part5 LLM部署技术" section 3 (no partial sum is
    dequantized: the whole K reduction stays in integers).
    """
    return np.asarray(x8, dtype=np.int64) @ np.asarray(w8, dtype=np.int64).T


def int_gemm_fp64(x8, w8):
    """Same product through an fp64 matmul of the integer values.

    Exact because every operand and every partial sum is an integer of
    magnitude below 2**53 (|acc| <= K * 127 * 121), so no rounding can occur
    in any summation order. Returned as int64.
    """
    a = np.asarray(x8, dtype=np.float64)
    b = np.asarray(w8, dtype=np.float64)
    return (a @ b.T).astype(np.int64)


def epilogue(acc, s_x, s1):
    """y[m, n] = acc[m, n] * s_x[m] * s1[n] in fp64 (scales applied once)."""
    acc = np.asarray(acc, dtype=np.float64)
    sx = np.asarray(s_x, dtype=np.float32).astype(np.float64)
    sw = np.asarray(s1, dtype=np.float16).astype(np.float64)
    return acc * sx[:, None] * sw[None, :]


def w4a8_linear(x, W, group=128):
    """Whole path on the CPU: quantize W and x, integer GEMM, epilogue."""
    wq = quantize_weights(W, group)
    w8 = dequantize_level2(wq["q4"], wq["s2"], wq["z"], group)
    x8, s_x = quantize_act(x)
    acc = int_gemm(x8, w8)
    return {"acc": acc, "y": epilogue(acc, s_x, wq["s1"]), "x8": x8, "s_x": s_x,
            "w8": w8, **wq}
