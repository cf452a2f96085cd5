"""Pins that tie the CPU oracle to facts fixed outside of it.

Each ``pin_*`` function takes an oracle namespace (the real ``oracle``
package, or a copy with a planted mistake) and raises AssertionError when
the oracle disagrees with:

* the hand-worked cases in golden/hand_cases.txt (exact rational derivation,
  see golden/derive_hand_cases.py);
* exhaustive enumerations (every level-2 group the protective range allows);
* textbook routines and brute force (pure-Python loops on tiny inputs,
  Python's round() on Fractions);
* closed-form error bounds and invariants of the definitions.

test_oracle.py runs every pin against the oracle; test_oracle_mutants.py
plants plausible mistakes in copies of the oracle and checks that each one
is caught by at least one pin.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.txt")


# --------------------------------------------------------------------------
def load_hand_cases(path=GOLDEN):
    rows = {}
    group = None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "group":
                group = int(parts[1])
                continue
            key, idx, vals = parts[0], int(parts[1]), parts[2:]
            rows.setdefault(key, {})[idx] = vals
    def mat(key, conv):
        d = rows[key]
        return [[conv(v) for v in d[i]] for i in sorted(d)]
    return {
        "group": group,
        "W": np.array(mat("w_row", float), dtype=np.float32),
        "s1": np.array([r[0] for r in mat("s1", float)], dtype=np.float64),
        "q8": np.array(mat("q8", int)),
        "s2": np.array(mat("s2", int)),
        "z": np.array(mat("z", int)),
        "q4": np.array(mat("q4", int)),
        "w8": np.array(mat("w8", int)),
        "X": np.array(mat("x_row", float), dtype=np.float16),
        "x8": np.array(mat("x8", int)),
        "s_x": np.array([r[0] for r in mat("s_x", float)], dtype=np.float64),
        "acc": np.array(mat("acc", int)),
        "y": np.array(mat("y", float), dtype=np.float64),
    }


def _exhaustive_groups(protect):
    """One row per (lo, hi) in [-protect, 0] x [0, protect]: the pair itself
    followed by every value of [-protect, protect] clipped into [lo, hi], so
    each row holds every code a group with that range can contain."""
    span = np.arange(-protect, protect + 1)
    rows = []
    for lo in range(-protect, 1):
        for hi in range(0, protect + 1):
            rows.append(np.concatenate([[lo, hi], np.clip(span, lo, hi)]))
    return np.array(rows, dtype=np.int64)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_hand_cases(O):
    """Every stage on the hand-worked rows equals the exact derivation."""
    h = load_hand_cases()
    G = h["group"]
    s1, q8 = O.level1_per_channel(h["W"])
    assert np.array_equal(s1.astype(np.float64), h["s1"]), (s1, h["s1"])
    assert np.array_equal(np.asarray(q8, np.int64), h["q8"]), q8
    q4, s2, z = O.level2_per_group(q8, G)
    assert np.array_equal(np.asarray(s2, np.int64), h["s2"]), s2
    assert np.array_equal(np.asarray(z, np.int64), h["z"]), z
    assert np.array_equal(np.asarray(q4, np.int64), h["q4"]), q4
    w8 = O.dequantize_level2(q4, s2, z, G)
    assert np.array_equal(np.asarray(w8, np.int64), h["w8"]), w8
    x8, s_x = O.quantize_act(h["X"])
    assert np.array_equal(np.asarray(x8, np.int64), h["x8"]), x8
    assert np.array_equal(np.asarray(s_x, np.float64), h["s_x"]), s_x
    acc = O.int_gemm(x8, w8)
    assert np.array_equal(np.asarray(acc, np.int64), h["acc"]), acc
    y = O.epilogue(acc, s_x, s1)
    np.testing.assert_allclose(y, h["y"], rtol=1e-15, atol=0)
    full = O.w4a8_linear(h["X"], h["W"], G)
    assert np.array_equal(np.asarray(full["acc"], np.int64), h["acc"])


def pin_range_invariant(O):
    """Protective range 119: every group the level-1 codes allow dequantizes
    inside INT8 and inside the byte lanes of the register-parallel unpack."""
    q8 = _exhaustive_groups(119)
    G = q8.shape[1]
    q4, s2, z = O.level2_per_group(q8, G)
    q4 = np.asarray(q4, np.int64)
    s2 = np.asarray(s2, np.int64)
    z = np.asarray(z, np.int64)
    w8 = np.asarray(O.dequantize_level2(q4, s2, z, G), np.int64)
    assert q4.min() >= 0 and q4.max() <= 15
    assert s2.min() >= 1 and s2.max() <= 16
    assert z.min() >= 0 and z.max() <= 15
    assert w8.min() >= -121 and w8.max() <= 121, (w8.min(), w8.max())
    assert (q4 * s2).max() <= 225
    bias = 128 - z * s2
    assert bias.min() >= 7 and bias.max() <= 128
    lane = q4 * s2 + bias  # the unsigned byte before the sign flip
    assert lane.min() >= 0 and lane.max() <= 255
    assert np.array_equal(lane - 128, w8)
    # rounding error of level 2 is at most half a step
    assert np.all(2 * np.abs(w8 - q8) <= s2)
    # zero is represented exactly in every group: the code z dequantizes to 0
    zero_codes = np.asarray(O.dequantize_level2(z, s2, z, 1), np.int64)
    assert np.all(zero_codes == 0)


def pin_range_120_overflows(O):
    """Negative control: one more level-1 code (R = 120) already lets a
    dequantized weight reach 128, outside INT8 -- so 119 is the largest
    protective range under these level-2 rules."""
    q8 = _exhaustive_groups(120)
    G = q8.shape[1]
    q4, s2, z = O.level2_per_group(q8, G)
    w8 = np.asarray(O.dequantize_level2(q4, s2, z, G), np.int64)
    assert w8.max() >= 128 or w8.min() <= -129


def pin_level2_brute_force(O):
    """Scale = smallest integer whose 16 levels span [lo, hi]; zero = the code
    nearest to -lo/s2 (ties to even); codes = nearest level -- found here by
    brute-force search over candidates with exact rationals."""
    rng = np.random.default_rng(1)
    lows = rng.integers(-119, 1, 300)
    highs = rng.integers(0, 120, 300)
    # include the corner pairs
    lows = np.concatenate([lows, [0, -119, 0, -119, -1, 0]])
    highs = np.concatenate([highs, [0, 119, 119, 0, 0, 1]])
    G = 8
    rows = []
    for lo, hi in zip(lows, highs):
        vals = rng.integers(lo, hi + 1, G - 2)
        rows.append(np.concatenate([[lo, hi], vals]))
    q8 = np.array(rows, dtype=np.int64)
    q4, s2, z = O.level2_per_group(q8, G)
    q4 = np.asarray(q4, np.int64)
    s2 = np.asarray(s2, np.int64)[:, 0]
    z = np.asarray(z, np.int64)[:, 0]
    for r, (lo, hi) in enumerate(zip(lows, highs)):
        lo, hi = int(lo), int(hi)
        want_s = next(s for s in range(1, 64) if 15 * s >= hi - lo)
        assert s2[r] == want_s, (lo, hi, s2[r], want_s)
        target = Fraction(-lo, want_s)
        best = min(range(16), key=lambda c: (abs(Fraction(c) - target), c % 2))
        assert z[r] == best, (lo, hi, z[r], best)
        for k in range(G):
            v = Fraction(int(q8[r, k]), want_s)
            code = min(range(-16, 32), key=lambda c: (abs(Fraction(c) - v), c % 2)) + best
            code = min(15, max(0, code))
            assert q4[r, k] == code, (lo, hi, q8[r, k], q4[r, k], code)


def pin_rne_matches_python_round(O):
    """The exact integer round-half-even equals Python's round() on
    Fractions (banker's rounding) over a full small range."""
    num = np.arange(-300, 301)
    for den in range(1, 21):
        got = np.asarray(O.rne_div(num, den), np.int64)
        want = np.array([round(Fraction(int(n), den)) for n in num])
        assert np.array_equal(got, want), den
        got_c = np.asarray(O.ceil_div(num, den), np.int64)
        want_c = np.array([-((-int(n)) // den) for n in num])
        assert np.array_equal(got_c, want_c), den


def pin_lossless_requantization(O):
    """A group whose level-1 codes already lie on a level-2 lattice {(c - z) s}
    that uses both end codes 0 and 15 is reproduced exactly, so progressive
    quantization of such a row equals per-channel INT8. (The group holding
    the row absmax +-119 cannot be on any lattice: 119 = 7 * 17 needs more
    than 15 steps, so that group is excluded from the comparison.)"""
    rng = np.random.default_rng(2)
    G = 16
    N, K = 12, 80
    q8 = np.zeros((N, K), np.int64)
    for n in range(N):
        q8[n, :G] = rng.integers(-119, 120, G)
        q8[n, 0] = 119 if n % 2 else -119  # the row absmax, in group 0
        for g in range(1, K // G):
            s = int(rng.integers(1, 8))
            z = int(rng.integers(0, 16))
            codes = rng.integers(0, 16, G)
            codes[0], codes[1] = 0, 15
            q8[n, g * G:(g + 1) * G] = (codes - z) * s
    scale = np.float32(2.0 ** -9)
    W = q8.astype(np.float32) * scale
    s1, q8b = O.level1_per_channel(W)
    assert np.all(s1.astype(np.float64) == float(scale))
    assert np.array_equal(np.asarray(q8b, np.int64), q8)
    q4, s2, z = O.level2_per_group(q8b, G)
    w8 = np.asarray(O.dequantize_level2(q4, s2, z, G), np.int64)
    assert np.array_equal(w8[:, G:], q8[:, G:])
    assert not np.array_equal(w8[:, 0], q8[:, 0])


def pin_identity_case(O):
    """Group scale 1 and zero 0: w8 equals the codes and the integer GEMM is
    the textbook int64 matrix product x8 @ q4^T (checked with literal Python
    loops on a non-square case to catch a transposed operand)."""
    rng = np.random.default_rng(3)
    M, K, N, G = 3, 8, 5, 4
    q4 = rng.integers(0, 16, (N, K))
    s2 = np.ones((N, K // G), np.int64)
    z = np.zeros((N, K // G), np.int64)
    w8 = np.asarray(O.dequantize_level2(q4, s2, z, G), np.int64)
    assert np.array_equal(w8, q4)
    z8 = np.full((N, K // G), 8)
    assert np.array_equal(np.asarray(O.dequantize_level2(q4, s2, z8, G), np.int64), q4 - 8)
    x8 = rng.integers(-127, 128, (M, K))
    acc = np.asarray(O.int_gemm(x8, w8), np.int64)
    assert acc.shape == (M, N)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == sum(int(x8[m, k]) * int(q4[n, k]) for k in range(K))


def pin_int_gemm_brute_force(O):
    """int_gemm and its fp64 twin equal a pure-Python triple loop, including
    at the overflow-relevant extremes (all codes +-127 x +-121)."""
    rng = np.random.default_rng(4)
    M, K, N = 4, 24, 6
    x8 = rng.integers(-127, 128, (M, K))
    w8 = rng.integers(-121, 122, (N, K))
    want = np.array([[sum(int(x8[m, k]) * int(w8[n, k]) for k in range(K))
                      for n in range(N)] for m in range(M)])
    assert np.array_equal(np.asarray(O.int_gemm(x8, w8), np.int64), want)
    assert np.array_equal(np.asarray(O.int_gemm_fp64(x8, w8), np.int64), want)
    # extreme magnitudes at the largest K of the workloads
    K = 24576
    x8 = np.full((2, K), 127)
    x8[1] = -127
    w8 = np.full((3, K), 121)
    w8[1] = -121
    w8[2, ::2] = -121
    big = np.asarray(O.int_gemm(x8, w8), np.int64)
    assert big[0, 0] == K * 127 * 121 and big[1, 0] == -K * 127 * 121
    assert big[0, 2] == 0
    assert np.array_equal(np.asarray(O.int_gemm_fp64(x8, w8), np.int64), big)
    # odd products whose running sums pass 2**24: exact only in wide types
    w8 = rng.integers(50, 61, (2, K)) * 2 + 1
    x8 = np.full((1, K), 127)
    x8[0, ::3] = 125
    want = [sum(int(a) * int(b) for a, b in zip(x8[0], w8[n])) for n in range(2)]
    assert list(np.asarray(O.int_gemm(x8, w8), np.int64)[0]) == want
    assert list(np.asarray(O.int_gemm_fp64(x8, w8), np.int64)[0]) == want


def pin_float_dequant_then_matmul(O):
    """Scaling once at the end equals dequantizing both operands to floats
    and multiplying in fp64 (brute-force float path), on a tiny case."""
    rng = np.random.default_rng(5)
    M, K, N, G = 3, 32, 4, 8
    W = (np.float32(0.02) * rng.standard_normal((N, K), dtype=np.float32))
    X = rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)
    res = O.w4a8_linear(X, W, G)
    xf = np.asarray(res["x8"], np.float64) * np.asarray(res["s_x"], np.float64)[:, None]
    wf = np.asarray(res["w8"], np.float64) * res["s1"].astype(np.float64)[:, None]
    want = np.array([[sum(xf[m, k] * wf[n, k] for k in range(K)) for n in range(N)]
                     for m in range(M)])
    np.testing.assert_allclose(res["y"], want, rtol=1e-12, atol=1e-15)


def pin_error_bounds(O):
    """Closed-form bounds on the representation error of each level."""
    rng = np.random.default_rng(6)
    N, K, G = 64, 512, 128
    W = (np.float32(0.02) * rng.standard_normal((N, K), dtype=np.float32))
    W[3] = 0.0                         # a zero channel
    W[5, :G] = np.abs(W[5, :G])        # an all-positive group
    W[6, G:2 * G] = -np.abs(W[6, G:2 * G])  # an all-negative group
    q = O.quantize_weights(W, G)
    s1 = q["s1"].astype(np.float64)
    q8 = np.asarray(q["q8"], np.int64)
    w8 = np.asarray(O.dequantize_level2(q["q4"], q["s2"], q["z"], G), np.int64)
    s2 = np.repeat(np.asarray(q["s2"], np.int64), G, axis=1)
    Wd = W.astype(np.float64)
    # level 1: half a step plus fp32 rounding of the quotient
    e1 = np.abs(q8 * s1[:, None] - Wd)
    assert np.all(e1 <= s1[:, None] * (0.5 + 1e-6) + 1e-30)
    # each nonzero row's absmax maps to +-119 exactly
    live = s1 > 0
    assert np.all(np.abs(q8[live]).max(axis=1) == 119)
    # zero channel
    assert s1[3] == 0 and np.all(q8[3] == 0) and np.all(np.asarray(q["q4"])[3] == 0)
    assert np.all(np.asarray(q["s2"])[3] == 1) and np.all(np.asarray(q["z"])[3] == 0)
    # one-signed groups: zero point at the end of the code range
    assert np.asarray(q["z"])[5, 0] == 0
    assert np.asarray(q["q4"])[6, G:2 * G].min() >= 0
    # both levels together
    e2 = np.abs(w8 * s1[:, None] - Wd)
    assert np.all(e2 <= s1[:, None] * (1 + s2) / 2 * (1 + 1e-6) + 1e-30)
    # activations: half a step, absmax maps to +-127, zero row
    X = rng.standard_normal((8, K), dtype=np.float32)
    X[:, 7] *= 20
    X[2] = 0
    X16 = X.astype(np.float16)
    x8, s_x = O.quantize_act(X16)
    x8 = np.asarray(x8, np.int64)
    s_x = np.asarray(s_x, np.float64)
    ea = np.abs(x8 * s_x[:, None] - X16.astype(np.float64))
    assert np.all(ea <= s_x[:, None] * (0.5 + 1e-5))
    rows = [m for m in range(8) if m != 2]
    assert np.all(np.abs(x8[rows]).max(axis=1) == 127)
    assert s_x[2] == 0 and np.all(x8[2] == 0)


def pin_scale_roundings(O):
    """s1 is the fp32 quotient absmax/119 rounded to fp16 (round-half-even,
    subnormals included) and s_x the fp32 quotient absmax/127: compared with
    an exact-rational rounding on random rows."""
    from golden.derive_hand_cases import fp16, fp32, round_half_even  # exact roundings
    rng = np.random.default_rng(7)
    N, K = 48, 16
    mags = np.float32(10.0) ** rng.uniform(-7, 1, N).astype(np.float32)
    W = (rng.standard_normal((N, K), dtype=np.float32) * mags[:, None]).astype(np.float32)
    s1, _ = O.level1_per_channel(W)
    for n in range(N):
        a = Fraction(float(np.max(np.abs(W[n]))))
        assert Fraction(float(s1[n])) == fp16(fp32(a / 119)), n
    X = (rng.standard_normal((N, K), dtype=np.float32) * 3).astype(np.float16)
    x8, s_x = O.quantize_act(X)
    for m in range(N):
        a = Fraction(float(np.max(np.abs(X[m].astype(np.float32)))))
        assert Fraction(float(s_x[m])) == fp32(a / 127), m
        inv = fp32(Fraction(127) / a)
        for k in range(K):
            code = round_half_even(fp32(Fraction(float(X[m, k])) * inv))
            assert int(x8[m, k]) == max(-127, min(127, code)), (m, k)


def pin_zero_padding_invariance(O):
    """Padding a group with zero codes changes neither its scale, its zero
    point nor the codes of the other entries (zero is always in the range)."""
    rng = np.random.default_rng(8)
    q8 = rng.integers(-119, 120, (50, 4))
    q8[:10] = np.abs(q8[:10])
    q8[10:20] = -np.abs(q8[10:20])
    a4, b4, c4 = O.level2_per_group(q8, 4)
    padded = np.concatenate([q8, np.zeros((50, 124), np.int64)], axis=1)
    a, b, c = O.level2_per_group(padded, 128)
    assert np.array_equal(np.asarray(b4), np.asarray(b))
    assert np.array_equal(np.asarray(c4), np.asarray(c))
    assert np.array_equal(np.asarray(a4), np.asarray(a)[:, :4])


PINS = [
    pin_hand_cases,
    pin_range_invariant,
    pin_range_120_overflows,
    pin_level2_brute_force,
    pin_rne_matches_python_round,
    pin_lossless_requantization,
    pin_identity_case,
    pin_int_gemm_brute_force,
    pin_float_dequant_then_matmul,
    pin_error_bounds,
    pin_scale_roundings,
    pin_zero_padding_invariance,
]
