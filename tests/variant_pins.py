"""Pins of the comparison-GEMM oracle (oracle/variants.py) to facts fixed
outside of it: exact rational derivations of the quantizers (Fractions with
explicit IEEE round-to-nearest-even, from golden/derive_hand_cases.py, which
does not use the oracle), pure-Python brute force on tiny inputs, a special
case that reduces to a textbook per-channel product, and closed-form
bounds. Each pin takes an oracle namespace so test_oracle_mutants.py can run
it against copies with planted mistakes.
"""
from __future__ import annotations

from fractions import Fraction as F

import numpy as np

from golden.derive_hand_cases import fp16, fp32, round_half_even


def _clamp(v, lo, hi):
    return max(lo, min(hi, v))


def _rng_case(seed, rows, k, zero_row=None, zero_group=None, group=None):
    rng = np.random.default_rng(seed)
    W = (0.02 * rng.standard_normal((rows, k))).astype(np.float32)
    if zero_row is not None:
        W[zero_row] = 0
    if zero_group is not None:
        r, g = zero_group
        W[r, g * group:(g + 1) * group] = 0
    return W


def pin_w8a8_exact(O):
    """Scales and codes equal the exact-rational derivation."""
    W = _rng_case(11, 5, 64, zero_row=3)
    W[1, 7] = -W[1].__abs__().max() * 1.0001            # a distinct absmax element
    s, q = O.w8a8_quantize_weights(W)
    for n in range(W.shape[0]):
        row = [F(float(v)) for v in W[n]]
        a = max(abs(v) for v in row)
        s_ref = fp16(fp32(a / 127))
        assert F(float(s[n])) == s_ref, (n, s[n], s_ref)
        for k, v in enumerate(row):
            want = 0 if s_ref == 0 else _clamp(round_half_even(fp32(v / s_ref)), -127, 127)
            assert int(q[n, k]) == want, (n, k, q[n, k], want)


def pin_w8a8_linear_brute(O):
    """acc by pure-Python loops over the oracle's own codes; y = acc s_x s."""
    rng = np.random.default_rng(12)
    W = (0.05 * rng.standard_normal((3, 32))).astype(np.float32)
    X = rng.standard_normal((2, 32)).astype(np.float16)
    r = O.w8a8_linear(X, W)
    for m in range(2):
        for n in range(3):
            acc = sum(int(r["x8"][m, k]) * int(r["q8"][n, k]) for k in range(32))
            assert int(r["acc"][m, n]) == acc
            y = F(acc) * F(float(r["s_x"][m])) * F(float(r["s"][n]))
            assert abs(F(float(r["y"][m, n])) - y) <= abs(y) * F(1, 2 ** 50)
    # the full INT8 range is used: every live row has a +-127 code
    s, q = O.w8a8_quantize_weights(W)
    assert np.all(np.abs(q).max(axis=1) == 127)


def pin_w4a4_exact(O):
    """Per-group weight and activation scales and codes equal the exact
    derivation, including an all-zero group and rounding ties."""
    G = 8
    W = _rng_case(13, 3, 32, zero_group=(2, 1), group=G)
    s_w, wq = O.w4a4_quantize_weights(W, G)
    for n in range(3):
        for g in range(4):
            grp = [F(float(v)) for v in W[n, g * G:(g + 1) * G]]
            a = max(abs(v) for v in grp)
            s_ref = fp16(fp32(a / 7))
            assert F(float(s_w[n, g])) == s_ref, (n, g)
            for i, v in enumerate(grp):
                want = 0 if s_ref == 0 else _clamp(round_half_even(fp32(v / s_ref)), -7, 7)
                assert int(wq[n, g * G + i]) == want, (n, g, i)
    # activations: one group whose products land on exact .5 ties
    X = np.array([[0.5, -1.5, 2.5, 7.0, 3.5, -0.5, 1.0, 0.0] + [0.0] * 8,
                  [1.0, 2.0, -3.0, 0.25, 0.125, 6.0, -7.0, 5.5] * 2], dtype=np.float16)
    xq, s_a = O.w4a4_quantize_act(X, G)
    for m in range(2):
        for g in range(2):
            grp = [F(float(v)) for v in X[m, g * G:(g + 1) * G]]
            a = max(abs(v) for v in grp)
            if a == 0:
                assert s_a[m, g] == 0 and not np.any(xq[m, g * G:(g + 1) * G])
                continue
            inv = fp32(F(7) / a)
            assert F(float(s_a[m, g])) == fp32(a / 7)
            for i, v in enumerate(grp):
                want = _clamp(round_half_even(fp32(v * inv)), -7, 7)
                assert int(xq[m, g * G + i]) == want, (m, g, i, xq[m, g * G + i], want)
    # the ties 0.5, 2.5, -0.5 (times 7/7 = 1) round to even
    assert list(xq[0, :8]) == [0, -2, 2, 7, 4, 0, 1, 0]
    # a group where multiplying by fp32(7/a) and dividing by fp32(a/7) give
    # different codes (-0.72607421875 * fp32(7/a) rounds to -3)
    X2 = np.array([[1.4521484375, 0.427734375, -0.1539306640625, -0.195556640625,
                    -0.72607421875, 0.87109375, -0.2998046875, 0.65478515625]], dtype=np.float16)
    xq2, _ = O.w4a4_quantize_act(X2, G)
    a = F(1.4521484375)
    inv = fp32(F(7) / a)
    want = [_clamp(round_half_even(fp32(F(float(v)) * inv)), -7, 7) for v in X2[0]]
    assert list(xq2[0]) == want == [7, 2, -1, -1, -3, 4, -1, 3]


def pin_w4a4_partial_sums_brute(O):
    rng = np.random.default_rng(14)
    xq = rng.integers(-7, 8, (2, 24))
    wq = rng.integers(-7, 8, (3, 24))
    P = O.w4a4_partial_sums(xq, wq, 8)
    for m in range(2):
        for n in range(3):
            for g in range(3):
                want = sum(int(xq[m, k]) * int(wq[n, k]) for k in range(8 * g, 8 * g + 8))
                assert int(P[m, n, g]) == want


def pin_w4a4_dequant_matmul(O):
    """y equals the fp64 product of the dequantized operands (the same sum
    regrouped), to rounding."""
    rng = np.random.default_rng(15)
    G = 16
    W = (0.02 * rng.standard_normal((5, 64))).astype(np.float32)
    X = rng.standard_normal((4, 64)).astype(np.float16)
    r = O.w4a4_linear(X, W, G)
    xd = r["xq"].astype(np.float64) * np.repeat(r["s_a"].astype(np.float64), G, axis=1)
    wd = r["wq"].astype(np.float64) * np.repeat(r["s_w"].astype(np.float64), G, axis=1)
    ref = xd @ wd.T
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-15)
    assert np.all(r["term_abs"] >= np.abs(r["y"]) * (1 - 1e-12))


def pin_w4a4_whole_row_group(O):
    """group = K: per-token x per-channel INT4, a textbook scaled integer
    product (acc = xq @ wq^T, then both scales)."""
    rng = np.random.default_rng(16)
    W = (0.02 * rng.standard_normal((3, 32))).astype(np.float32)
    X = rng.standard_normal((2, 32)).astype(np.float16)
    r = O.w4a4_linear(X, W, 32)
    acc = r["xq"].astype(np.int64) @ r["wq"].astype(np.int64).T
    ref = acc * r["s_a"][:, 0].astype(np.float64)[:, None] * r["s_w"][:, 0].astype(np.float64)[None, :]
    assert np.allclose(r["y"], ref, rtol=1e-13, atol=0)


def pin_w4a4_bounds(O):
    """|x - q s| <= s/2 (plus fp32/fp16 rounding of the scale), the group
    absmax maps to +-7, codes stay in [-7, 7]."""
    rng = np.random.default_rng(17)
    G = 32
    X = rng.standard_normal((3, 128)).astype(np.float16)
    xq, s_a = O.w4a4_quantize_act(X, G)
    xf = X.astype(np.float64)
    sa = np.repeat(s_a.astype(np.float64), G, axis=1)
    assert np.all(np.abs(xq) <= 7)
    assert np.all(np.abs(xf - xq * sa) <= sa * (0.5 + 1e-5))
    am = np.abs(xf).reshape(3, 4, G).argmax(axis=2)
    for m in range(3):
        for g in range(4):
            assert abs(int(xq[m, g * G + am[m, g]])) == 7
    W = (0.02 * rng.standard_normal((4, 128))).astype(np.float32)
    s_w, wq = O.w4a4_quantize_weights(W, G)
    sw = np.repeat(s_w.astype(np.float64), G, axis=1)
    # fp16 rounding of the scale moves the absmax code at most to 7 (clamped)
    assert np.all(np.abs(wq) <= 7)
    assert np.all(np.abs(W - wq * sw) <= sw * (0.5 + 7 * 2.0 ** -11) + 1e-12)


def pin_w4a16_exact(O):
    """Scales, zeros, codes and fp16 dequantized weights equal the exact
    derivation, including a one-signed group and an all-zero group."""
    G = 8
    W = _rng_case(18, 3, 32, zero_group=(1, 2), group=G)
    W[2, 0:8] = np.abs(W[2, 0:8]) + np.float32(0.01)       # all positive: lo = 0
    q, s, z = O.w4a16_quantize_weights(W, G)
    w16 = O.w4a16_dequantize(q, s, z, G)
    for n in range(3):
        for g in range(4):
            grp = [F(float(v)) for v in W[n, g * G:(g + 1) * G]]
            lo, hi = min(F(0), min(grp)), max(F(0), max(grp))
            s_ref = fp16(fp32(fp32(hi - lo) / 15))
            assert F(float(s[n, g])) == s_ref, (n, g)
            if s_ref == 0:
                assert z[n, g] == 0 and not np.any(q[n, g * G:(g + 1) * G])
                continue
            z_ref = _clamp(round_half_even(fp32(-lo / s_ref)), 0, 15)
            assert int(z[n, g]) == z_ref, (n, g)
            for i, v in enumerate(grp):
                q_ref = _clamp(round_half_even(fp32(v / s_ref)) + z_ref, 0, 15)
                assert int(q[n, g * G + i]) == q_ref, (n, g, i)
                assert F(float(w16[n, g * G + i])) == fp16((q_ref - z_ref) * s_ref)


def pin_w4a16_linear_brute(O):
    """y and term_abs by pure-Python loops over the fp16 values."""
    rng = np.random.default_rng(19)
    W = (0.05 * rng.standard_normal((3, 16))).astype(np.float32)
    X = rng.standard_normal((2, 16)).astype(np.float16)
    r = O.w4a16_linear(X, W, 8)
    for m in range(2):
        for n in range(3):
            terms = [F(float(X[m, k])) * F(float(r["w16"][n, k])) for k in range(16)]
            assert abs(F(float(r["y"][m, n])) - sum(terms)) <= F(1, 2 ** 40)
            assert abs(F(float(r["term_abs"][m, n])) - sum(abs(t) for t in terms)) <= F(1, 2 ** 40)


def pin_w4a16_bounds(O):
    """|w - w16| <= s/2 plus fp16 rounding for weights inside [lo, hi];
    codes in [0, 15]; the zero code reproduces 0 up to rounding."""
    rng = np.random.default_rng(20)
    W = (0.02 * rng.standard_normal((4, 256))).astype(np.float32)
    q, s, z = O.w4a16_quantize_weights(W, 128)
    w16 = O.w4a16_dequantize(q, s, z, 128).astype(np.float64)
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    assert q.max() <= 15
    assert np.all(np.abs(W - w16) <= sf * 0.5 * (1 + 2.0 ** -8) + np.abs(W) * 2.0 ** -10)


VARIANT_PINS = [pin_w8a8_exact, pin_w8a8_linear_brute, pin_w4a4_exact,
                pin_w4a4_partial_sums_brute, pin_w4a4_dequant_matmul, pin_w4a4_whole_row_group,
                pin_w4a4_bounds, pin_w4a16_exact, pin_w4a16_linear_brute, pin_w4a16_bounds]
