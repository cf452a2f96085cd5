"""INT32 accumulators at the largest K the GEMM entry points accept, with the
operands that make them largest.

A weight row of one constant value quantizes (level 1) to 119 everywhere;
level 2 then gives every group of 128 the scale 8, the zero 0 and the code
15 (119 / 8 = 14.875 rounds up), so every dequantized weight is 120 (-120
for a negative row: zero 15, code 0). An activation row of one constant
value quantizes to 127 everywhere. At K = QOQ_MAX_GEMM_K = 139648 every
accumulator is then +-127 * 120 * K = +-2 128 235 520, 99.1 % of 2^31 - 1:
a kernel that summed in a narrower type, added a bias before the sum, or let
a split-K partial or the cross-wave sum wrap would be off. Each kernel
family (forced through the "gemm" tuning key), the default plans at
several token counts and the one-call linear path must give the oracle's
accumulators bit for bit and the fp16 output within 2e-3. The W8A8
comparison GEMM gets the same treatment at its own limit.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import variants as ovar

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
K_MAX = 139648
N = 256
Y_RTOL = 2e-3
Y_FLOOR = 2.0 ** -14


def _operands(M):
    """W rows +-0.02 alternating by channel, X rows +-1 alternating by token."""
    W = np.where(np.arange(N)[:, None] % 2 == 0, 0.02, -0.02).astype(np.float32) * np.ones(
        (1, K_MAX), np.float32)
    X = np.where(np.arange(M)[:, None] % 2 == 0, 1.0, -1.0).astype(np.float16) * np.ones(
        (1, K_MAX), np.float16)
    return W, X


_ref = {}


def _oracle():
    """The oracle on the two distinct token rows (every even row equals row 0,
    every odd row row 1); checked against the closed form first."""
    if "r" not in _ref:
        W, X = _operands(2)
        r = oracle.w4a8_linear(X, W)
        extreme = 127 * 120 * K_MAX
        assert extreme < 2 ** 31
        signs = np.where((np.arange(2)[:, None] + np.arange(N)[None, :]) % 2 == 0, 1, -1)
        assert np.array_equal(r["acc"], signs * extreme)
        _ref["r"] = r
    return _ref["r"]


_dev = {}


def _device_case(M):
    if M not in _dev:
        W, X = _operands(M)
        pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
        x = torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV)
        _dev[M] = (pw, x)
    return _dev[M]


def _check(M, y, acc):
    r = _oracle()
    rows = np.arange(M) % 2
    ref_acc = r["acc"][rows]
    ref_y = r["y"][rows]
    acc_h = acc.cpu().numpy().astype(np.int64)
    assert np.array_equal(acc_h, ref_acc), f"accumulators differ at K={K_MAX}, M={M}"
    yh = y.cpu().numpy().astype(np.float64)
    err = np.abs(yh - ref_y) / np.maximum(np.abs(ref_y), Y_FLOOR)
    assert err.max() <= Y_RTOL, f"y max relative error {err.max():.3e}"


@pytest.fixture(autouse=True)
def _clear_tuning():
    yield
    qoq.clear_tuning()


@pytest.mark.parametrize("M", [1, 16, 64, 256])
def test_default_plan_at_max_k(M):
    pw, x = _device_case(M)
    x8, s_x = qoq.quantize_act(x)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True, workspace=qoq.Workspace(DEV))
    torch.cuda.synchronize()
    _check(M, y, acc)


@pytest.mark.parametrize("M", [8, 64])
def test_linear_path_at_max_k(M):
    pw, x = _device_case(M)
    y, acc = qoq.w4a8_linear(x, pw, acc_debug=True, workspace=qoq.Workspace(DEV))
    torch.cuda.synchronize()
    _check(M, y, acc)


# one configuration of every family, and the split-K forms (partial sums of
# up to ~1.1e9 each, added by the second kernel)
FORCED = [
    (16, "decode,1,1,8,2"),
    (64, "decode,2,2,8,4"),
    (64, "lds,4,1,8,4"),
    (64, "lds,4,1,8,4,4"),
    (16, "lds,1,2,8,2,2"),
    (64, "tile32,2,1,4,2,4"),
    (64, "tile32,2,1,4,2,4,3"),
    (64, "ksplit,2,1,8,4"),
    (256, "ksplit,2,2,4,3"),
    (256, "wide,8,1,8,3,1"),
    (256, "wide,8,1,8,3,1,2"),
    (64, "stream,2,1,8,4,8"),
    (16, "generic,1,2"),
]


@pytest.mark.parametrize("M,cfg", FORCED, ids=[f"{c}@M{m}" for m, c in FORCED])
def test_family_at_max_k(M, cfg):
    pw, x = _device_case(M)
    x8, s_x = qoq.quantize_act(x)
    qoq.set_tuning("gemm", cfg)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True, workspace=qoq.Workspace(DEV))
    torch.cuda.synchronize()
    _check(M, y, acc)


# The W8A8 comparison GEMM keeps 8-bit weights over [-127, 127], so it stops
# at K = 133120 (127 * 127 * K < 2^31): constant rows give 127 on both sides
# and accumulators of +-2 147 092 480, 99.98 % of 2^31 - 1.
K_W8A8 = 133120


@pytest.mark.parametrize("M", [16, 256])
def test_w8a8_at_its_max_k(M):
    W = np.where(np.arange(N)[:, None] % 2 == 0, 0.02, -0.02).astype(np.float32) * np.ones(
        (1, K_W8A8), np.float32)
    X = np.where(np.arange(M)[:, None] % 2 == 0, 1.0, -1.0).astype(np.float16) * np.ones(
        (1, K_W8A8), np.float16)
    r = ovar.w8a8_linear(X[:2], W)
    extreme = 127 * 127 * K_W8A8
    assert extreme < 2 ** 31
    signs = np.where((np.arange(2)[:, None] + np.arange(N)[None, :]) % 2 == 0, 1, -1)
    assert np.array_equal(r["acc"], signs * extreme)
    packed, s = qoq.w8a8_pack_weights(torch.from_numpy(W).to(DEV))
    x8, s_x = qoq.quantize_act(torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV))
    y, acc = qoq.w8a8_gemm(x8, s_x, packed, s, N, acc_debug=True)
    torch.cuda.synchronize()
    rows = np.arange(M) % 2
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), r["acc"][rows])
    yh = y.cpu().numpy().astype(np.float64)
    ref_y = r["y"][rows]
    err = np.abs(yh - ref_y) / np.maximum(np.abs(ref_y), Y_FLOOR)
    assert err.max() <= Y_RTOL, f"y max relative error {err.max():.3e}"
