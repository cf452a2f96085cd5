"""Activation quantization + W4A8 GEMM captured in a HIP graph.

Serving loops replay the decode step as a graph. The captured step must give,
on every replay, exactly what the same calls give eagerly on the same inputs
(both are deterministic integer paths followed by one fp16 rounding), with
eager work and synchronizations between replays, and the eager result must
match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from act_layout import act_rows

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (M, K, N): a decode-family shape, a shared-activation shape (N > 8192) and a
# 32x32-tile shape (M > 64)
SHAPES = [(8, 1024, 1040), (32, 512, 8208), (100, 640, 208)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_graph_replays_match_eager(M, K, N):
    print(f"\n[gpu-case] graph M={M} K={K} N={N}", flush=True)
    W, _, _ = wl.make_inputs(1, K, N, seed=11 + N)
    pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
    xs = []
    for r in range(4):
        _, X, _ = wl.make_inputs(M, K, 16, seed=100 * r + M)
        xs.append(X)

    def dev_half(X):
        return torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV)

    x_static = torch.empty((M, K), dtype=torch.float16, device=DEV)
    x8 = qoq.empty_act(M, K, DEV)
    s_x = torch.empty(M, dtype=torch.float32, device=DEV)
    y = torch.empty((M, N), dtype=torch.float16, device=DEV)

    def step():
        qoq.quantize_act(x_static, out=(x8, s_x))
        qoq.w4a8_gemm(x8, s_x, pw, y=y)

    x_static.copy_(dev_half(xs[0]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r, X in enumerate(xs):
        xd = dev_half(X)
        # eager reference on separate buffers
        e8, es = qoq.quantize_act(xd)
        ey, eacc = qoq.w4a8_gemm(e8, es, pw, acc_debug=True)
        torch.cuda.synchronize()
        # graph replay on the static buffers
        y.fill_(0)
        x_static.copy_(xd)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(act_rows(x8, M), act_rows(e8, M)), f"replay {r}: x8 differs from eager"
        assert torch.equal(s_x, es), f"replay {r}: s_x differs from eager"
        assert torch.equal(y, ey), f"replay {r}: y differs from eager"
        if r == 0:
            ref = oracle.w4a8_linear(X, W)
            assert np.array_equal(eacc.cpu().numpy().astype(np.int64), ref["acc"])
            yy = ey.cpu().numpy().astype(np.float64)
            err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
            assert err.max() <= 2e-3


def test_graph_replay_after_workspace_grows():
    """A graph captured with a Workspace keeps writing its split-K partial
    sums into the buffer it captured: a later eager call that needs more
    bytes grows the Workspace, the superseded buffer stays alive, and the
    replay (with new tensors allocated in between) still matches eager."""
    (Ms, Ks, Ns), (Mb, Kb, Nb) = (128, 8192, 1024), (64, 16384, 4096)
    qoq.set_tuning("gemm", None)
    small = qoq.qoq_gemm_workspace_bytes(Ms, Ns, Ks)
    big = qoq.qoq_gemm_workspace_bytes(Mb, Nb, Kb)
    assert 0 < small < big, (small, big)
    print(f"\n[gpu-case] graph + workspace growth {small} -> {big} bytes", flush=True)
    Ws, Xs, _ = wl.make_inputs(Ms, Ks, Ns, seed=41)
    Wb, Xb, _ = wl.make_inputs(Mb, Kb, Nb, seed=43)
    pws = qoq.pack_weights(torch.from_numpy(Ws).to(DEV))
    pwb = qoq.pack_weights(torch.from_numpy(Wb).to(DEV))
    xs = torch.from_numpy(Xs.view(np.uint16)).view(torch.float16).to(DEV)
    xb = torch.from_numpy(Xb.view(np.uint16)).view(torch.float16).to(DEV)
    ws = qoq.Workspace(DEV)
    x8, s_x = qoq.quantize_act(xs)
    y = torch.empty((Ms, Ns), dtype=torch.float16, device=DEV)

    def step():
        qoq.w4a8_gemm(x8, s_x, pws, y=y, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                     # sizes the workspace before the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    captured = ws.buf.data_ptr()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ey, _ = qoq.w4a8_gemm(x8, s_x, pws, acc_debug=True)

    # a bigger call grows the workspace; allocations that could reuse a
    # freed buffer are made and filled before the replay
    b8, bs = qoq.quantize_act(xb)
    yb = qoq.w4a8_gemm(b8, bs, pwb, workspace=ws)
    assert ws.buf.data_ptr() != captured and ws.buf.numel() >= big
    assert any(r.data_ptr() == captured for r in ws.retired)
    fillers = [torch.full((small,), 0x5A, dtype=torch.uint8, device=DEV) for _ in range(4)]
    torch.cuda.synchronize()
    for r in range(3):
        y.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ey), f"replay {r} after growth differs from eager"
        assert all(bool((f == 0x5A).all()) for f in fillers), "a replay wrote into a new tensor"
    ebig, _ = qoq.w4a8_gemm(b8, bs, pwb, acc_debug=True)
    assert torch.equal(yb, ebig)
