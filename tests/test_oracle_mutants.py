"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutant is the oracle's own source with one textual change (a dropped
term, a wrong sign, a wrong rounding, a transposed or truncated operand, a
wrong constant), executed as a fresh module on the CPU. The real oracle is
never modified. A mutant that survives every pin means the pins have a blind
spot, so the test fails.
"""
import os
import types

import pytest

from oracle_pins import PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "qoq_oracle.py")

MUTANTS = [
    # level 1
    ("protect 127", "PROTECT = 119", "PROTECT = 127"),
    ("level-1 truncation", "codes = np.clip(np.rint(ratio)", "codes = np.clip(np.trunc(ratio)"),
    ("level-1 scale kept fp32", "s1 = s1_f32.astype(np.float16)", "s1 = s1_f32"),
    ("level-1 no clamp", "np.clip(np.rint(ratio), -protect, protect)", "np.rint(ratio)"),
    ("level-1 absmax as max", "absmax = np.max(np.abs(W), axis=1)", "absmax = np.max(W, axis=1)"),
    # level 2
    ("range without zero (lo)", "lo = np.minimum(0, grouped.min(axis=2))", "lo = grouped.min(axis=2)"),
    ("range without zero (hi)", "hi = np.maximum(0, grouped.max(axis=2))", "hi = grouped.max(axis=2)"),
    ("scale rounds instead of ceil", "s2 = np.maximum(1, ceil_div(hi - lo, Q4_MAX))",
     "s2 = np.maximum(1, rne_div(hi - lo, Q4_MAX))"),
    ("scale floor", "s2 = np.maximum(1, ceil_div(hi - lo, Q4_MAX))",
     "s2 = np.maximum(1, np.floor_divide(hi - lo, Q4_MAX))"),
    ("scale over 16 levels", "s2 = np.maximum(1, ceil_div(hi - lo, Q4_MAX))",
     "s2 = np.maximum(1, ceil_div(hi - lo, Q4_MAX + 1))"),
    ("zero floor", "z = rne_div(-lo, s2)", "z = np.floor_divide(-lo, s2)"),
    ("zero sign", "z = rne_div(-lo, s2)", "z = rne_div(lo, s2)"),
    ("codes without zero point", "rne_div(grouped, s2[:, :, None]) + z[:, :, None]",
     "rne_div(grouped, s2[:, :, None])"),
    ("codes floor", "rne_div(grouped, s2[:, :, None]) + z[:, :, None]",
     "np.floor_divide(grouped, s2[:, :, None]) + z[:, :, None]"),
    # rounding helper
    ("rne rounds half up", "round_up = (twice > den) | ((twice == den) & (quo % 2 != 0))",
     "round_up = twice >= den"),
    ("ceil is floor", "return -np.floor_divide(-num, den)", "return np.floor_divide(num, den)"),
    # dequantization
    ("zero term not scaled", "zero_term = (z * s2)[:, :, None]", "zero_term = z[:, :, None]"),
    ("zero term added", "return (scaled - zero_term)", "return (scaled + zero_term)"),
    ("scale dropped", "scaled = q4.reshape(n_rows, k // group, group) * s2[:, :, None]",
     "scaled = q4.reshape(n_rows, k // group, group) * 1"),
    # activations
    ("act 128 levels", "ACT_MAX = 127", "ACT_MAX = 128"),
    ("act divides by scale", "prod = xf[live] * inv[:, None]",
     "prod = xf[live] / (absmax[live] / np.float32(ACT_MAX))[:, None]"),
    ("act truncation", "x8[live] = np.clip(np.rint(prod)", "x8[live] = np.clip(np.trunc(prod)"),
    ("act scale inverted", "s_x[live] = absmax[live] / np.float32(ACT_MAX)",
     "s_x[live] = np.float32(ACT_MAX) / absmax[live]"),
    ("act absmax over tokens", "absmax = np.max(np.abs(xf), axis=1) if",
     "absmax = np.max(np.abs(xf), axis=0)[:xf.shape[0]] if"),
    # GEMM
    ("gemm int16 accumulate", "return np.asarray(x8, dtype=np.int64) @ np.asarray(w8, dtype=np.int64).T",
     "return (np.asarray(x8, dtype=np.int16) @ np.asarray(w8, dtype=np.int16).T).astype(np.int64)"),
    ("gemm drops last k", "return np.asarray(x8, dtype=np.int64) @ np.asarray(w8, dtype=np.int64).T",
     "return np.asarray(x8, dtype=np.int64)[:, :-1] @ np.asarray(w8, dtype=np.int64)[:, :-1].T"),
    ("gemm fp32", "return (a @ b.T).astype(np.int64)",
     "return (a.astype(np.float32) @ b.astype(np.float32).T).astype(np.int64)"),
    # epilogue
    ("epilogue drops token scale", "return acc * sx[:, None] * sw[None, :]", "return acc * sw[None, :]"),
    ("epilogue drops channel scale", "return acc * sx[:, None] * sw[None, :]", "return acc * sx[:, None]"),
]


def _mutant_module(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _mutant_module(old, new)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"mutant '{name}' survived every pin"


def test_unmutated_copy_passes():
    mod = _mutant_module("PROTECT = 119", "PROTECT = 119")
    for pin in PINS:
        pin(mod)
