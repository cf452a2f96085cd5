"""Planted mistakes in copies of the comparison-GEMM oracle must each fail
at least one of its pins (same scheme as test_oracle_mutants.py)."""
import os
import types

import pytest

from variant_pins import VARIANT_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "variants.py")
IMPORT = "from .qoq_oracle import level1_per_channel, quantize_act, int_gemm, epilogue"

MUTANTS = [
    ("w8 protective range", "W8_MAX = 127", "W8_MAX = 119"),
    ("int4 range 8", "INT4_MAX = 7", "INT4_MAX = 8"),
    ("int4 range 15", "INT4_MAX = 7", "INT4_MAX = 15"),
    ("w4 weight truncation", "q[live] = np.clip(np.rint(ratio)", "q[live] = np.clip(np.trunc(ratio)"),
    ("w4 weight scale kept fp32",
     "s_w = (absmax / np.float32(INT4_MAX)).astype(np.float16)",
     "s_w = (absmax / np.float32(INT4_MAX))"),
    ("w4 weight absmax signed", "absmax = np.max(np.abs(g), axis=2)                       # exact",
     "absmax = np.max(g, axis=2)                       # exact"),
    ("a4 divides by scale", "prod = g[live] * inv[:, None]",
     "prod = g[live] / (absmax[live] / np.float32(INT4_MAX))[:, None]"),
    ("a4 truncation", "q[live] = np.clip(np.rint(prod)", "q[live] = np.clip(np.trunc(prod)"),
    ("a4 scale inverted", "s_a[live] = absmax[live] / np.float32(INT4_MAX)",
     "s_a[live] = np.float32(INT4_MAX) / absmax[live]"),
    ("partial sums pair wrong groups", 'return np.einsum("mgk,ngk->mng", a, b)',
     'return np.einsum("mgk,ngk->mng", a, b[:, ::-1])'),
    ("partial sums drop last input", 'return np.einsum("mgk,ngk->mng", a, b)',
     'return np.einsum("mgk,ngk->mng", a[:, :, :-1], b[:, :, :-1])'),
    ("y drops weight scale", "* s_w.astype(np.float64)[None, :, :]", "* 1.0"),
    ("w4a16 range without zero", "lo = np.minimum(np.float32(0), g.min(axis=2))", "lo = g.min(axis=2)"),
    ("w4a16 scale over 16 levels", "s = ((hi - lo) / np.float32(15)).astype(np.float16)",
     "s = ((hi - lo) / np.float32(16)).astype(np.float16)"),
    ("w4a16 scale kept fp32", "s = ((hi - lo) / np.float32(15)).astype(np.float16)",
     "s = ((hi - lo) / np.float32(15))"),
    ("w4a16 zero sign", "np.rint(-lo[live] / s_back[live])", "np.rint(lo[live] / s_back[live])"),
    ("w4a16 codes without zero", "q[live] = np.clip(codes + z[live][:, None], 0, 15)",
     "q[live] = np.clip(codes, 0, 15)"),
    ("w4a16 dequant adds zero", "prod = (q - np.asarray(z, dtype=np.int64)[:, :, None])",
     "prod = (q + np.asarray(z, dtype=np.int64)[:, :, None])"),
    ("w4a16 dequant kept exact", "return prod.reshape(n_rows, -1).astype(np.float16)",
     "return prod.reshape(n_rows, -1)"),
    ("y drops token scale", "scale = s_a.astype(np.float64)[:, None, :]",
     "scale = np.ones_like(s_a, dtype=np.float64)[:, None, :]"),
]


def _mutant_module(old, new):
    src = open(SRC_PATH).read()
    assert src.count(IMPORT) == 1
    src = src.replace(IMPORT, IMPORT.replace("from .qoq_oracle", "from oracle.qoq_oracle"))
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mod = types.ModuleType("variants_mutant")
    exec(compile(src.replace(old, new), "variants_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_variant_mutant_is_caught(name, old, new):
    mod = _mutant_module(old, new)
    caught = []
    for pin in VARIANT_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"mutant '{name}' survived every pin"


def test_unmutated_copy_passes():
    mod = _mutant_module("W8_MAX = 127", "W8_MAX = 127")
    for pin in VARIANT_PINS:
        pin(mod)
