"""Planted mistakes in copies of the KV4 attention oracle must each fail at
least one of its pins (same scheme as test_oracle_mutants.py)."""
import os
import types

import pytest

from kv4_pins import KV4_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "kv4.py")
IMPORT = "from .variants import w4a16_quantize_weights"

MUTANTS = [
    ("keys multiplied by lambda", "ksm = kf / np.asarray(lam, dtype=np.float16)",
     "ksm = kf * np.asarray(lam, dtype=np.float16)"),
    ("values smoothed too", "vc, vs, vz = kv4_quantize(vf)", "vc, vs, vz = kv4_quantize(ksm * 0 + vf / 2)"),
    ("query not smoothed", "return (qf * lam_h[None, :, :]).astype(np.float16)",
     "return qf.astype(np.float16)"),
    ("query divided by lambda", "return (qf * lam_h[None, :, :]).astype(np.float16)",
     "return (qf / lam_h[None, :, :]).astype(np.float16)"),
    ("query lambda by head modulo", "lam_h = np.repeat(", "lam_h = np.tile("),
    ("smoothing factor without square root", "lam = np.sqrt(a).astype(np.float16)",
     "lam = a.astype(np.float16)"),
    ("smoothing factor zero for empty channel", "lam[a == 0] = np.float16(1.0)",
     "lam[a == 0] = np.float16(0.0)"),
    ("scores scaled by 1 / D", "sc = (k @ q) / np.sqrt(D)", "sc = (k @ q) / D"),
    ("scores unscaled", "sc = (k @ q) / np.sqrt(D)", "sc = (k @ q)"),
    ("grouped heads by modulo", "hk = h // group", "hk = h % kh.shape[2]"),
    ("length off by one", "n = int(lens[b])", "n = int(lens[b]) + 1"),
    ("softmax not normalized", "o[b, h] = (w @ v) / w.sum()", "o[b, h] = (w @ v)"),
    ("dequantization adds zero", "return (c - zz) *", "return (c + zz) *"),
]


def _mutant_module(old, new):
    src = open(SRC_PATH).read()
    assert src.count(IMPORT) == 1
    src = src.replace(IMPORT, IMPORT.replace("from .variants", "from oracle.variants"))
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mod = types.ModuleType("kv4_mutant")
    exec(compile(src.replace(old, new), "kv4_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_kv4_mutant_is_caught(name, old, new):
    mod = _mutant_module(old, new)
    caught = []
    for pin in KV4_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError, OverflowError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"mutant '{name}' survived every pin"


def test_unmutated_copy_passes():
    mod = _mutant_module("hk = h // group", "hk = h // group")
    for pin in KV4_PINS:
        pin(mod)
