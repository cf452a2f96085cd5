"""GPU path (libqoq through its C ABI) against the CPU oracle, element by
element on the same seeded inputs.

Bars: codes, scales, activation codes and INT32 accumulators bit-exact; the
fp16 output within a relative error of 2e-3 of the oracle's fp64 value
(denominator floored at 2**-14, the smallest normal fp16).

Small cases are compared in full; the full-size workloads are compared on
sampled output channels and tokens (level 1 and level 2 act on one channel
at a time and activation quantization on one token at a time, so the oracle
can quantize only the sampled rows) with the launch configuration the
benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from act_layout import act_rows
from guard import Guarded, GuardedWorkspace

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
Y_RTOL = 2e-3
Y_FLOOR = 2.0 ** -14


def _announce(*what):
    print("\n[gpu-case]", *what, flush=True)


def gpu_run(W, X, canonical=True, acc_debug=True):
    """Pack, quantize and multiply on the GPU with every output (x8, s_x, y,
    the accumulators, the workspace) inside guard bands that are checked
    after each launch."""
    M, K = X.shape
    N = W.shape[0]
    Wd = torch.from_numpy(W).to(DEV)
    Xd = torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV)
    pw = qoq.pack_weights(Wd, canonical=canonical)
    gx8 = Guarded(((M + 15) // 16, K // 16, 16, 16), torch.int8, DEV)
    gsx = Guarded((M,), torch.float32, DEV)
    x8, s_x = qoq.quantize_act(Xd, out=(gx8.t, gsx.t))
    gx8.check("x8")
    gsx.check("s_x")
    gy = Guarded((M, N), torch.float16, DEV)
    gacc = Guarded((M, N), torch.int32, DEV) if acc_debug else None
    ws = GuardedWorkspace(qoq.qoq_gemm_workspace_bytes(M, N, K), DEV)
    out = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=gacc.t if acc_debug else False, y=gy.t,
                        workspace=ws)
    y, acc = out if acc_debug else (out, None)
    torch.cuda.synchronize()
    gy.check("y")
    ws.check()
    if acc_debug:
        gacc.check("acc_debug")
    return pw, x8, s_x, y, acc


def check_y(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref) / np.maximum(np.abs(y_ref), Y_FLOOR)
    assert np.all(np.isfinite(y_gpu))
    assert err.max() <= Y_RTOL, f"max rel err {err.max():.3e}"
    return err.max()


def check_canonical(pw, W_rows, rows):
    """Sampled (or all) rows of the GPU canonical output vs the oracle."""
    q = oracle.quantize_weights(W_rows)
    s1 = pw.s1.view(torch.int16)[rows].cpu().numpy().view(np.float16)
    assert np.array_equal(s1.view(np.uint16), q["s1"].view(np.uint16)), "s1"
    assert np.array_equal(pw.q4[rows].cpu().numpy(), q["q4"]), "q4"
    assert np.array_equal(pw.s2[rows].cpu().numpy().astype(np.int64), np.asarray(q["s2"], np.int64)), "s2"
    assert np.array_equal(pw.z[rows].cpu().numpy(), q["z"]), "z"
    return q


def full_check(W, X):
    pw, x8, s_x, y, acc = gpu_run(W, X)
    ref = oracle.w4a8_linear(X, W)
    rows = torch.arange(W.shape[0], device=DEV)
    check_canonical(pw, W, rows)
    assert np.array_equal(act_rows(x8, X.shape[0]), ref["x8"]), "x8"
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), ref["s_x"].view(np.uint32)), "s_x"
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"]), "acc"
    return check_y(y.cpu().numpy().astype(np.float64), ref["y"])


def sampled_check(W, X, pw, x8, s_x, y, acc, n_cols=96, n_rows=64, seed=0):
    M, K = X.shape
    N = W.shape[0]
    rng = np.random.default_rng(seed + 1000)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N),
                                     rng.choice(N, n_cols, replace=False)]))
    if M <= 256:
        toks = np.arange(M)
    else:
        toks = np.unique(np.concatenate([[0, M - 1], rng.choice(M, n_rows, replace=False)]))
    q = check_canonical(pw, W[cols], torch.from_numpy(cols).to(DEV))
    w8 = oracle.dequantize_level2(q["q4"], q["s2"], q["z"], wl.GROUP)
    x8_ref, sx_ref = oracle.quantize_act(X[toks])
    assert np.array_equal(act_rows(x8, M)[toks], x8_ref), "x8"
    assert np.array_equal(s_x.cpu().numpy()[toks].view(np.uint32), sx_ref.view(np.uint32)), "s_x"
    acc_ref = oracle.int_gemm_fp64(x8_ref, w8)
    t_idx = torch.from_numpy(toks).to(DEV)
    c_idx = torch.from_numpy(cols).to(DEV)
    acc_gpu = acc.index_select(0, t_idx).index_select(1, c_idx).cpu().numpy().astype(np.int64)
    assert np.array_equal(acc_gpu, acc_ref), f"acc mismatch at {np.argwhere(acc_gpu != acc_ref)[:5]}"
    y_gpu = y.index_select(0, t_idx).index_select(1, c_idx).cpu().numpy().astype(np.float64)
    return check_y(y_gpu, oracle.epilogue(acc_ref, sx_ref, q["s1"]))


# ---------------------------------------------------------------------------
# small cases, full comparison
# ---------------------------------------------------------------------------
def test_tiny_workload_full():
    w = wl.WORKLOADS["tiny"]
    shape = w.shapes[0]
    W, X, _ = wl.make_case(w, shape, w.Ms[0])
    _announce("tiny full", shape)
    full_check(W, X)


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (3, 384, 48), (17, 1152, 80), (33, 256, 272),
                                   (65, 640, 144), (100, 1024, 1040), (255, 512, 208),
                                   (300, 768, 400), (64, 4096, 4096)])
def test_ragged_shapes_full(M, K, N):
    _announce("ragged", M, K, N)
    W, X, _ = wl.make_inputs(M, K, N, seed=M * 7 + N)
    full_check(W, X)


def test_degenerate_rows_and_channels():
    """Zero tokens, zero channels, one-signed groups, a huge outlier."""
    M, K, N = 20, 512, 64
    W, X, _ = wl.make_inputs(M, K, N, seed=11)
    X[3] = 0
    X[7, 5] = np.float16(60000.0)
    W[9] = 0
    W[10, :128] = np.abs(W[10, :128])
    W[11, 128:256] = -np.abs(W[11, 128:256])
    W[12, 300] = 1.0  # one large weight dominates its channel
    _announce("degenerate")
    full_check(W, X)


def test_identity_canonical_packing():
    """s2 = 1, z = 0 packed from canonical codes: the GEMM must equal the
    textbook int64 product x8 @ q4^T; z = 8 gives signed int4 weights."""
    M, K, N = 37, 1024, 96
    rng = np.random.default_rng(5)
    q4 = rng.integers(0, 16, (N, K), dtype=np.uint8)
    s1 = (rng.uniform(0.5, 2.0, N) / 64).astype(np.float16)
    _, X, _ = wl.make_inputs(M, K, 16, seed=5)
    Xd = torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV)
    x8, s_x = qoq.quantize_act(Xd)
    x8_h = act_rows(x8, M)
    x8_ref, sx_ref = oracle.quantize_act(X)
    assert np.array_equal(x8_h, x8_ref)
    for zero in (0, 8):
        _announce("identity", zero)
        s2 = np.ones((N, K // 128), np.int8)
        z = np.full((N, K // 128), zero, np.uint8)
        pw = qoq.pack_canonical(torch.from_numpy(q4).to(DEV), torch.from_numpy(s2).to(DEV),
                                torch.from_numpy(z).to(DEV), torch.from_numpy(s1).to(DEV))
        y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
        want = x8_ref.astype(np.int64) @ (q4.astype(np.int64) - zero).T
        assert np.array_equal(acc.cpu().numpy().astype(np.int64), want)
        check_y(y.cpu().numpy().astype(np.float64), oracle.epilogue(want, sx_ref, s1))


def test_offsets_beyond_2_31():
    """The largest shapes: 2^32 weights (2 GiB of packed nibbles), so byte
    offsets pass 2^31 and the plan takes the 64-bit generic kernel. Codes are
    packed from canonical form (s2 = 1, random zeros) generated on the GPU;
    the oracle checks sampled output channels for M = 1 and a ragged M = 20."""
    N, K = 32768, 131072
    assert qoq.qoq_packed_weight_bytes(N, K) > (1 << 31)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    q4 = torch.randint(0, 16, (N, K), dtype=torch.uint8, device=DEV, generator=g)
    z = torch.randint(0, 16, (N, K // 128), dtype=torch.uint8, device=DEV, generator=g)
    s2 = torch.ones((N, K // 128), dtype=torch.int8, device=DEV)
    s1 = (torch.rand(N, device=DEV, generator=g) * 0.01 + 0.001).to(torch.float16)
    pw = qoq.pack_canonical(q4, s2, z, s1)
    rng = np.random.default_rng(13)
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 46, replace=False)]))
    ci = torch.from_numpy(cols).to(DEV)
    w8 = oracle.dequantize_level2(q4.index_select(0, ci).cpu().numpy(),
                                  s2.index_select(0, ci).cpu().numpy(),
                                  z.index_select(0, ci).cpu().numpy(), 128)
    s1_s = s1.index_select(0, ci).cpu().numpy()
    del q4
    for M in (1, 20):
        _announce("offsets beyond 2^31", M, K, N)
        _, X, _ = wl.make_inputs(M, K, 16, seed=M)
        x8, s_x = qoq.quantize_act(torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV))
        y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
        torch.cuda.synchronize()
        x8_ref, sx_ref = oracle.quantize_act(X)
        assert np.array_equal(act_rows(x8, M), x8_ref)
        want = x8_ref.astype(np.int64) @ w8.astype(np.int64).T
        got = acc.index_select(1, ci).cpu().numpy().astype(np.int64)
        assert np.array_equal(got, want)
        check_y(y.index_select(1, ci).cpu().numpy().astype(np.float64),
                oracle.epilogue(want, sx_ref, s1_s))


def test_hand_cases_padded():
    """The hand-worked groups, zero-padded to 128 inputs (padding with zero
    changes no group parameter), through the GPU path."""
    from oracle_pins import load_hand_cases
    h = load_hand_cases()
    G = h["group"]
    n_rows, k = h["W"].shape
    W = np.zeros((16, 128 * (k // G)), np.float32)
    for g in range(k // G):
        W[:n_rows, 128 * g:128 * g + G] = h["W"][:, G * g:G * (g + 1)]
    X = np.zeros((h["X"].shape[0], 128 * (k // G)), np.float16)
    for g in range(k // G):
        X[:, 128 * g:128 * g + G] = h["X"][:, G * g:G * (g + 1)]
    _announce("hand cases")
    pw, x8, s_x, y, acc = gpu_run(W, X)
    s1 = pw.s1.cpu().numpy().astype(np.float64)[:n_rows]
    assert np.array_equal(s1, h["s1"])
    assert np.array_equal(s_x.cpu().numpy().astype(np.float64), h["s_x"])
    assert np.array_equal(acc.cpu().numpy()[:, :n_rows].astype(np.int64), h["acc"])
    assert np.all(acc.cpu().numpy()[:, n_rows:] == 0)
    q4 = pw.q4.cpu().numpy()[:n_rows]
    for g in range(k // G):
        assert np.array_equal(q4[:, 128 * g:128 * g + G], h["q4"][:, G * g:G * (g + 1)])


def test_empty_batch_is_a_no_op():
    W, _, _ = wl.make_inputs(1, 256, 32, seed=1)
    pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
    x8 = qoq.empty_act(0, 256, DEV)
    s_x = torch.empty(0, dtype=torch.float32, device=DEV)
    y = qoq.w4a8_gemm(x8, s_x, pw)
    assert y.shape == (0, 32)
    x8b, sxb = qoq.quantize_act(torch.empty((0, 256), dtype=torch.float16, device=DEV))
    assert x8b.shape == (0, 16, 16, 16) and sxb.shape == (0,)


# shapes whose plan keeps split-K partial sums in the workspace: the default
# plans of the shared-activation and 32x32 families, and forced splits of the
# shared-activation, wide-tile and weight-streaming families
SPLIT_CASES = [(64, 16384, 4096, None), (128, 8192, 1024, None),
               (64, 2560, 528, "lds,4,1,4,2,3"), (300, 2560, 528, "wide,4,2,8,4,1,2"),
               (40, 2560, 1040, "stream,2,1,8,4,8,3"), (64, 16384, 4096, None)]


def test_workspace_is_reusable(monkeypatch):
    """One workspace (with guard bands) serves split-K calls of different
    shapes and families back to back: each call writes all of its partial
    sums before reading them, so stale sums of the previous call never leak
    into the result, and nothing is written outside the workspace."""
    need = []
    for (M, K, N, cfg) in SPLIT_CASES:
        if cfg:
            qoq.set_tuning("gemm", cfg)
        else:
            qoq.set_tuning("gemm", None)
        need.append(qoq.qoq_gemm_workspace_bytes(M, N, K))
    assert all(b > 0 for b in need), need
    ws = GuardedWorkspace(max(need), DEV)
    for (M, K, N, cfg) in SPLIT_CASES:
        if cfg:
            qoq.set_tuning("gemm", cfg)
        else:
            qoq.set_tuning("gemm", None)
        _announce("workspace reuse", M, K, N, cfg)
        W, X, _ = wl.make_inputs(M, K, N, seed=3 + M + N)
        pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
        x8, s_x = qoq.quantize_act(torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV))
        y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True, workspace=ws)
        ws.check()
        q = oracle.quantize_weights(W)
        w8 = oracle.dequantize_level2(q["q4"], q["s2"], q["z"], wl.GROUP)
        x8_ref, sx_ref = oracle.quantize_act(X)
        acc_ref = oracle.int_gemm_fp64(x8_ref, w8)
        assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
        check_y(y.cpu().numpy().astype(np.float64), oracle.epilogue(acc_ref, sx_ref, q["s1"]))


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------
CASES = [(key, shape.name, M) for key in wl.ORDER[1:] for shape in wl.WORKLOADS[key].shapes
         for M in wl.WORKLOADS[key].Ms]
COMMON_TILE_CASES = {("llama3_8b", "qkv", 256), ("llama3_8b", "gate_up", 256), ("prefill", "prefill", 4096),
                     ("qwen15_72b", "gate_up", 1024), ("qwen15_72b", "down", 1024)}


@pytest.mark.parametrize("key,shape_name,M", CASES, ids=[f"{k}-{s}-M{m}" for k, s, m in CASES])
def test_workload_full_size_all_outputs(key, shape_name, M, monkeypatch):
    """Every benchmarked layer at full size under the GEMM's default plan
    (the decode, shared-activation, K-split, 32x32 and wide tile families,
    K split into ranges through the workspace where the plan does; the 1-
    and 8-token decode layers also run fused, tests/test_gpu_linear.py),
    every output: the INT32 accumulators bit-exact against the oracle's
    exact GEMM (fp64 BLAS on the integer codes, exact below 2^53) and y
    within the tolerance."""
    w = wl.WORKLOADS[key]
    shape = next(s for s in w.shapes if s.name == shape_name)
    qoq.set_tuning("gemm", None)
    split = qoq.qoq_gemm_workspace_bytes(M, shape.N, shape.K) > 0
    _announce("all outputs", key, shape_name, M, shape.K, shape.N, "split K" if split else "")
    W, X, _ = wl.make_case(w, shape, M)
    pw, x8, s_x, y, acc = gpu_run(W, X, canonical=False)
    q = oracle.quantize_weights(W)
    w8 = oracle.dequantize_level2(q["q4"], q["s2"], q["z"], wl.GROUP)
    del W
    x8_ref, sx_ref = oracle.quantize_act(X)
    assert np.array_equal(act_rows(x8, M), x8_ref), "x8"
    acc_ref = oracle.int_gemm_fp64(x8_ref, w8)
    got = acc.cpu().numpy()
    bad = np.argwhere(got != acc_ref)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at {bad[:4]}"
    err = check_y(y.cpu().numpy().astype(np.float64), oracle.epilogue(acc_ref, sx_ref, q["s1"]))
    print(f"[gpu-case] ok, all {M * shape.N} outputs, max rel err {err:.2e}", flush=True)


def test_split_k_plans_among_the_workloads():
    """The all-outputs cases include split-K plans (partial sums through the
    workspace and the split-K epilogue kernel)."""
    split = [(k, s, m) for k, s, m in CASES
             if qoq.qoq_gemm_workspace_bytes(m, next(x for x in wl.WORKLOADS[k].shapes if x.name == s).N,
                                             next(x for x in wl.WORKLOADS[k].shapes if x.name == s).K) > 0]
    assert ("qwen15_72b", "down", 1024) in split and ("qwen15_72b", "down", 64) in split, split


@pytest.mark.parametrize("key,shape_name,M", CASES, ids=[f"{k}-{s}-M{m}" for k, s, m in CASES])
def test_workload_full_size_sampled(key, shape_name, M, monkeypatch):
    w = wl.WORKLOADS[key]
    shape = next(s for s in w.shapes if s.name == shape_name)
    _announce("workload", key, shape_name, M, shape.K, shape.N)
    qoq.set_tuning("gemm", None)
    W, X, _ = wl.make_case(w, shape, M)
    pw, x8, s_x, y, acc = gpu_run(W, X)
    err = sampled_check(W, X, pw, x8, s_x, y, acc)
    print(f"[gpu-case] ok max rel err {err:.2e}", flush=True)
    if (key, shape_name, M) in COMMON_TILE_CASES:
        # the benchmark's format comparison also times the common 64 x 128 tile
        qoq.set_tuning("gemm", "tile32,2,1,2,2,4")
        y2, acc2 = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
        torch.cuda.synchronize()
        sampled_check(W, X, pw, x8, s_x, y2, acc2)
