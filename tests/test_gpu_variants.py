"""The comparison GEMMs (W8A8 per-channel; W4A4 per-group with partial-sum
scaling; W4A16 weight-only) against their oracle: codes, scales and zeros
bit-exact (read through the documented layouts), W8A8 INT32 accumulators
bit-exact, W8A8 fp16 output within the QoQ tolerance, W4A4 and W4A16 fp16
output within the error bound of their fp32 accumulation; the W4A16 in-loop
dequantization bit-exact through one-hot activations."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from act_layout import act_rows
from variant_layout import w4_codes_scales, w4a16_codes_scales_zeros, w8_codes, x4_codes_scales

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPES = [(1, 128, 16), (5, 640, 208), (37, 384, 48), (64, 2048, 528), (100, 640, 208),
          (300, 1152, 528), (257, 256, 1040)]
W8_CONFIGS = ["4,2,2,2,4", "4,2,2,1,8", "4,1,2,1,8", "2,2,2,2,4", "2,1,4,2,4", "1,1,4,3,4",
              "2,1,2,2,4"]
W4_CONFIGS = ["2,1,2,2,4", "2,1,2,1,8", "1,1,2,3,4", "2,2,2,2,4"]
W16_CONFIGS = ["2,1,2,2,4", "2,2,2,2,4", "4,1,2,1,8", "1,1,2,3,4", "4,2,2,1,8"]


def _half(X):
    return torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV)


def _w8(M, K, N, monkeypatch, cfg=None):
    W, X, _ = wl.make_inputs(M, K, N, seed=3 * M + K + N)
    qoq.set_tuning("variant", None)
    packed, s = qoq.w8a8_pack_weights(torch.from_numpy(W).to(DEV))
    x8, s_x = qoq.quantize_act(_half(X))
    if cfg:
        qoq.set_tuning("variant", cfg)
    print(f"\n[gpu-case] w8a8 cfg={cfg} M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w8a8_gemm(x8, s_x, packed, s, N, acc_debug=True)
    torch.cuda.synchronize()
    ref = oracle.w8a8_linear(X, W)
    assert np.array_equal(w8_codes(packed.cpu().numpy(), N, K), ref["q8"]), "codes"
    assert np.array_equal(s.cpu().numpy().view(np.uint16), ref["s"].view(np.uint16)), "scales"
    assert np.array_equal(act_rows(x8, M), ref["x8"])
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"]), "acc"
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3


def _w4(M, K, N, monkeypatch, cfg=None):
    W, X, _ = wl.make_inputs(M, K, N, seed=5 * M + K + N)
    qoq.set_tuning("variant", None)
    packed = qoq.w4a4_pack_weights(torch.from_numpy(W).to(DEV))
    act = qoq.w4a4_quantize_act(_half(X))
    if cfg:
        qoq.set_tuning("variant", cfg)
    print(f"\n[gpu-case] w4a4 cfg={cfg} M={M} K={K} N={N}", flush=True)
    y = qoq.w4a4_gemm(act, M, K, packed, N)
    torch.cuda.synchronize()
    ref = oracle.w4a4_linear(X, W)
    codes, sc = w4_codes_scales(packed.cpu().numpy(), N, K)
    assert np.array_equal(codes, ref["wq"]), "weight codes"
    assert np.array_equal(sc.view(np.uint16), ref["s_w"].view(np.uint16)), "weight scales"
    xq, s_a = x4_codes_scales(act.cpu().numpy(), M, K)
    assert np.array_equal(xq, ref["xq"]), "activation codes"
    assert np.array_equal(s_a.view(np.uint32), ref["s_a"].view(np.uint32)), "activation scales"
    # fp32 accumulation of K/128 scaled partial sums, then one fp16 rounding
    ng = K // 128
    yy = y.cpu().numpy().astype(np.float64)
    tol = 2.0 ** -11 * np.abs(ref["y"]) + (ng + 2) * 2.0 ** -22 * ref["term_abs"] + 2.0 ** -24
    bad = np.abs(yy - ref["y"]) > tol
    assert not bad.any(), f"{bad.sum()} outputs outside the bound, first at {np.argwhere(bad)[:3]}"


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w8a8_default(M, K, N, monkeypatch):
    _w8(M, K, N, monkeypatch)


@pytest.mark.parametrize("cfg", W8_CONFIGS)
def test_w8a8_every_config(cfg, monkeypatch):
    for (M, K, N) in [(37, 384, 48), (300, 1152, 528)]:
        _w8(M, K, N, monkeypatch, cfg)


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w4a4_default(M, K, N, monkeypatch):
    _w4(M, K, N, monkeypatch)


@pytest.mark.parametrize("cfg", W4_CONFIGS)
def test_w4a4_every_config(cfg, monkeypatch):
    for (M, K, N) in [(37, 384, 48), (300, 1152, 528)]:
        _w4(M, K, N, monkeypatch, cfg)


def test_w4a4_zero_groups(monkeypatch):
    W, X, _ = wl.make_inputs(20, 512, 64, seed=9)
    W[3, 128:256] = 0
    X[7, 256:384] = 0
    X[11] = 0
    qoq.set_tuning("variant", None)
    packed = qoq.w4a4_pack_weights(torch.from_numpy(W).to(DEV))
    act = qoq.w4a4_quantize_act(_half(X))
    y = qoq.w4a4_gemm(act, 20, 512, packed, 64)
    ref = oracle.w4a4_linear(X, W)
    tol = 2.0 ** -11 * np.abs(ref["y"]) + 6 * 2.0 ** -22 * ref["term_abs"] + 2.0 ** -24
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - ref["y"]) <= tol)
    assert torch.all(y[11] == 0)


def _w16_check_weights(packed, ref, N, K):
    q, sc, z = w4a16_codes_scales_zeros(packed.cpu().numpy(), N, K)
    assert np.array_equal(q, ref["q"]), "weight codes"
    assert np.array_equal(sc.view(np.uint16), ref["s"].view(np.uint16)), "weight scales"
    assert np.array_equal(z, ref["z"]), "zeros"


def _w16(M, K, N, monkeypatch, cfg=None, W=None, X=None):
    if W is None:
        W, X, _ = wl.make_inputs(M, K, N, seed=7 * M + K + N)
    qoq.set_tuning("variant", None)
    packed = qoq.w4a16_pack_weights(torch.from_numpy(W).to(DEV))
    if cfg:
        qoq.set_tuning("variant", cfg)
    print(f"\n[gpu-case] w4a16 cfg={cfg} M={M} K={K} N={N}", flush=True)
    y = qoq.w4a16_gemm(_half(X), packed, N)
    torch.cuda.synchronize()
    ref = oracle.w4a16_linear(X, W)
    _w16_check_weights(packed, ref, N, K)
    # exact fp16 products summed in fp32 (K terms), then one fp16 rounding
    yy = y.cpu().numpy().astype(np.float64)
    tol = 2.0 ** -11 * np.abs(ref["y"]) + (K + 2) * 2.0 ** -23 * ref["term_abs"] + 2.0 ** -24
    bad = np.abs(yy - ref["y"]) > tol
    assert not bad.any(), f"{bad.sum()} outputs outside the bound, first at {np.argwhere(bad)[:3]}"
    return y, ref


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w4a16_default(M, K, N, monkeypatch):
    _w16(M, K, N, monkeypatch)


@pytest.mark.parametrize("cfg", W16_CONFIGS)
def test_w4a16_every_config(cfg, monkeypatch):
    for (M, K, N) in [(37, 384, 48), (300, 1152, 528)]:
        _w16(M, K, N, monkeypatch, cfg)


@pytest.mark.parametrize("cfg", [None] + W16_CONFIGS)
def test_w4a16_dequantization_exact(cfg, monkeypatch):
    """One-hot rows select single weights: y[m, n] = w16[n, m] with nothing to
    round, so the in-loop dequantization is compared bit for bit."""
    K, N = 640, 208
    M = K
    W, _, _ = wl.make_inputs(1, K, N, seed=23)
    X = np.eye(M, K, dtype=np.float16)
    y, ref = _w16(M, K, N, monkeypatch, cfg, W=W, X=X)
    assert np.array_equal(y.cpu().numpy(), ref["w16"].T), "dequantized weights differ"


def test_w4a16_zero_groups_and_empty(monkeypatch):
    W, X, _ = wl.make_inputs(20, 512, 64, seed=29)
    W[3, 128:256] = 0
    W[5] = 0
    X[11] = 0
    y, ref = _w16(20, 512, 64, monkeypatch, W=W, X=X)
    assert torch.all(y[11] == 0) and torch.all(y[:, 5] == 0)
    assert ref["s"][3, 1] == 0 and ref["z"][3, 1] == 0
    packed = qoq.w4a16_pack_weights(torch.from_numpy(W).to(DEV))
    e = qoq.w4a16_gemm(torch.empty((0, 512), dtype=torch.float16, device=DEV), packed, 64)
    assert e.shape == (0, 64)


# ---------------------------------------------------------------------------
# full-size workload shapes, sampled outputs, in the launch configurations the
# benchmark times (each variant's default plan and the common 64 x 128 tile)
# ---------------------------------------------------------------------------
FULL = [("llama3_8b", "qkv", 256), ("llama3_8b", "gate_up", 256), ("prefill", "prefill", 4096),
        ("qwen15_72b", "gate_up", 1024), ("qwen15_72b", "down", 1024)]


def _sample(M, N, seed):
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(N, 64, replace=False)]))
    toks = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 48), replace=False)]))
    return toks, cols


def _pick(t, toks, cols):
    ti = torch.from_numpy(toks).to(DEV)
    ci = torch.from_numpy(cols).to(DEV)
    return t.index_select(0, ti).index_select(1, ci).cpu().numpy()


@pytest.mark.parametrize("key,sname,M", FULL, ids=[f"{k}-{s}-{m}" for k, s, m in FULL])
def test_variants_full_size_sampled(key, sname, M, monkeypatch):
    w = wl.WORKLOADS[key]
    shp = next(s for s in w.shapes if s.name == sname)
    K, N = shp.K, shp.N
    W, X, _ = wl.make_case(w, shp, M)
    toks, cols = _sample(M, N, seed=M + N)
    Ws, Xs = W[cols], X[toks]
    ref8 = oracle.w8a8_linear(Xs, Ws)
    ref4 = oracle.w4a4_linear(Xs, Ws)
    ref16 = oracle.w4a16_linear(Xs, Ws)
    qoq.set_tuning("variant", None)
    Wd = torch.from_numpy(W).to(DEV)
    del W
    xd = _half(X)
    p8, s8 = qoq.w8a8_pack_weights(Wd)
    p4 = qoq.w4a4_pack_weights(Wd)
    p16 = qoq.w4a16_pack_weights(Wd)
    del Wd
    x8, s_x = qoq.quantize_act(xd)
    a4 = qoq.w4a4_quantize_act(xd)
    ng = K // 128
    for cfg in (None, "2,1,2,2,4"):
        if cfg:
            qoq.set_tuning("variant", cfg)
        print(f"\n[gpu-case] variants full {key} {sname} M={M} cfg={cfg}", flush=True)
        y8, acc8 = qoq.w8a8_gemm(x8, s_x, p8, s8, N, acc_debug=True)
        y4 = qoq.w4a4_gemm(a4, M, K, p4, N)
        y16 = qoq.w4a16_gemm(xd, p16, N)
        torch.cuda.synchronize()
        assert np.array_equal(_pick(acc8, toks, cols).astype(np.int64), ref8["acc"]), f"w8a8 acc {cfg}"
        yy = _pick(y8, toks, cols).astype(np.float64)
        assert (np.abs(yy - ref8["y"]) / np.maximum(np.abs(ref8["y"]), 2.0 ** -14)).max() <= 2e-3
        yy = _pick(y4, toks, cols).astype(np.float64)
        tol = 2.0 ** -11 * np.abs(ref4["y"]) + (ng + 2) * 2.0 ** -22 * ref4["term_abs"] + 2.0 ** -24
        assert not (np.abs(yy - ref4["y"]) > tol).any(), f"w4a4 {cfg}"
        yy = _pick(y16, toks, cols).astype(np.float64)
        tol = 2.0 ** -11 * np.abs(ref16["y"]) + (K + 2) * 2.0 ** -23 * ref16["term_abs"] + 2.0 ** -24
        assert not (np.abs(yy - ref16["y"]) > tol).any(), f"w4a16 {cfg}"
        qoq.set_tuning("variant", None)
