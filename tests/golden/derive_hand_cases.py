"""Derive the hand-worked cases in hand_cases.txt by exact rational arithmetic.

This script does NOT use the oracle or NumPy: it restates each quantizer step
with Python's Fraction and an explicit IEEE round-to-nearest-even to a given
binary format, so the stored values are an independent derivation. Run it to
regenerate the fixture:

    python tests/golden/derive_hand_cases.py > tests/golden/hand_cases.txt

Steps followed (pages: the velog notes on QServe, "Methods" sections, and the
abstract; readings of the unstated details are in the design notes):
level 1 per-channel symmetric INT8 inside the protective range 119 with an
FP16 scale; level 2 per-group UINT4 with integer scale and zero; per-token
symmetric INT8 activations; dequantization by subtraction after
multiplication; integer GEMM; one scaling at the end.
"""
from __future__ import annotations

from fractions import Fraction as F
import math


def round_half_even(q: F) -> int:
    fl = math.floor(q)
    rem = q - fl
    if rem > F(1, 2):
        return fl + 1
    if rem < F(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def to_binary(q: F, mant_bits: int, min_exp: int) -> F:
    """Round q to the nearest value with mant_bits fraction bits (RNE),
    subnormals below 2**min_exp; no overflow handling (values are small)."""
    if q == 0:
        return F(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a))
    # fix floating log2 inaccuracy
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    ulp = F(2) ** (e - mant_bits)
    return sign * round_half_even(a / ulp) * ulp


def fp32(q: F) -> F:
    return to_binary(q, 23, -126)


def fp16(q: F) -> F:
    return to_binary(q, 10, -14)


def clamp(v, lo, hi):
    return max(lo, min(hi, v))


def level1(row):
    a = max(abs(v) for v in row)
    s1 = fp16(fp32(a / 119))
    if s1 == 0:
        return s1, [0] * len(row)
    return s1, [clamp(round_half_even(fp32(v / s1)), -119, 119) for v in row]


def level2(q8, G):
    q4, s2s, zs = [], [], []
    for g in range(0, len(q8), G):
        grp = q8[g:g + G]
        lo, hi = min(0, min(grp)), max(0, max(grp))
        s2 = max(1, -((-(hi - lo)) // 15))
        z = round_half_even(F(-lo, s2))
        s2s.append(s2)
        zs.append(z)
        q4 += [clamp(round_half_even(F(v, s2)) + z, 0, 15) for v in grp]
    return q4, s2s, zs


def act(row):
    a = max(abs(v) for v in row)
    if a == 0:
        return [0] * len(row), F(0)
    inv = fp32(F(127) / a)
    return [clamp(round_half_even(fp32(v * inv)), -127, 127) for v in row], fp32(a / 127)


def fmt(vals):
    return " ".join(str(v) for v in vals)


def main():
    G = 4
    # weights: three output channels of 8 inputs (two groups of 4 each)
    W = [[F("0.5"), F(-1), F("0.25"), F(0), F("0.03"), F("0.06"), F("-0.02"), F("0.01")],
         [F("0.125"), F("0.25"), F("0.375"), F("0.5"), F("-0.0625"), F(0), F("0.1875"), F("0.4375")],
         # a tiny channel: its scale lands among the fp16 subnormals, so the
         # absmax code exceeds the protective range before the clamp
         [F(119 * 7, 5) * F(1, 2 ** 24) * c for c in
          (F(1), F(-1, 2), F(1, 3), F(0), F(-1), F(3, 4), F(1, 8), F(-5, 8))]]
    # the decimal literals above are first rounded to fp32, as the inputs are
    W = [[fp32(v) for v in r] for r in W]
    # activations: four tokens (fp16 inputs, exactly representable)
    X = [[F(1), F(-2), F(1, 2), F(0), F(3), F(-3), F(1, 4), F(3, 2)],
         [F(0)] * 8,
         [F(-7, 8), F(1, 16), F(5), F(-5, 2), F(1, 8), F(9, 4), F(-1), F(11, 4)],
         # x = absmax/2 sits on a code boundary where multiplying by the fp32
         # reciprocal and dividing by the fp32 scale round differently
         [F(2110, 1024), F(1055, 1024), F(-1055, 1024), F(1, 2), F(-1, 8), F(3, 2), F(0),
          F(-2110, 1024)]]
    print("# hand-worked cases; derived by tests/golden/derive_hand_cases.py with exact rationals")
    print(f"group {G}")
    w8_rows, s1s = [], []
    for n, row in enumerate(W):
        s1, q8 = level1(row)
        q4, s2, z = level2(q8, G)
        w8 = [(q4[k] * s2[k // G]) - z[k // G] * s2[k // G] for k in range(len(row))]
        w8_rows.append(w8)
        s1s.append(s1)
        print(f"w_row {n} " + fmt(float(v) for v in row))
        print(f"s1 {n} {float(s1)!r}")
        print(f"q8 {n} " + fmt(q8))
        print(f"s2 {n} " + fmt(s2))
        print(f"z {n} " + fmt(z))
        print(f"q4 {n} " + fmt(q4))
        print(f"w8 {n} " + fmt(w8))
    x8_rows, sxs = [], []
    for m, row in enumerate(X):
        x8, sx = act(row)
        x8_rows.append(x8)
        sxs.append(sx)
        print(f"x_row {m} " + fmt(float(v) for v in row))
        print(f"x8 {m} " + fmt(x8))
        print(f"s_x {m} {float(sx)!r}")
    for m in range(len(X)):
        accs = [sum(a * b for a, b in zip(x8_rows[m], w8_rows[n])) for n in range(len(W))]
        ys = [float(accs[n] * sxs[m] * s1s[n]) for n in range(len(W))]
        print(f"acc {m} " + fmt(accs))
        print(f"y {m} " + fmt(repr(v) for v in ys))


if __name__ == "__main__":
    main()
