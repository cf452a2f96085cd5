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
