"""The one-call entry point (activation quantization + W4A8 GEMM) against
the oracle and against the two-call path.

Small M runs the fused kernel, which quantizes the tokens inside the GEMM;
its codes, accumulators and fp16 outputs must equal the two-call path's bit
for bit, and the accumulators the oracle's. Larger shapes run the two-call
path through the workspace.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (M, K, N): one to sixteen tokens, group counts that do and do not fill the
# waves, column counts that fill no tile
FUSED = [(1, 128, 16), (1, 4096, 4096), (8, 4096, 4096), (5, 640, 208), (8, 1152, 400), (8, 8192, 528),
         (3, 2048, 1040), (4, 512, 512), (2, 384, 48),
         # 5-12 tokens with two column blocks per workgroup (more than 16e6
         # values quantized, or 9-12 tokens past 4096 columns; odd block
         # counts: the last workgroup's second block lies past N), 8 or 16
         # waves; 9 tokens on 4096 columns with one block
         (8, 4096, 8208), (6, 8192, 5648), (9, 4096, 4096), (10, 4096, 6144),
         (11, 4096, 4112), (12, 8192, 1040)]
# (the fused kernel also takes up to 16 tokens when forced)
FORCED = FUSED + [(16, 8192, 528), (13, 2048, 1040), (9, 512, 512), (12, 640, 16)]
TWO_CALL = [(17, 1024, 208), (64, 4096, 4096), (8, 14336, 272), (100, 640, 400), (16, 512, 512)]


def _half(X):
    return torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV)


def _check(M, K, N, monkeypatch, cfg=None):
    W, X, _ = wl.make_inputs(M, K, N, seed=7 * M + K + N)
    pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
    xd = _half(X)
    qoq.set_tuning("gemm", None)
    x8, s_x = qoq.quantize_act(xd)
    y2, acc2 = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    if cfg is not None:
        qoq.set_tuning("gemm", cfg)
    print(f"\n[gpu-case] linear cfg={cfg} M={M} K={K} N={N}", flush=True)
    y1, acc1 = qoq.w4a8_linear(xd, pw, acc_debug=True)
    torch.cuda.synchronize()
    ref = oracle.w4a8_linear(X, W)
    assert np.array_equal(acc1.cpu().numpy().astype(np.int64), ref["acc"]), "acc vs oracle"
    assert torch.equal(acc1, acc2), "acc vs two-call path"
    assert torch.equal(y1, y2), "y vs two-call path"
    yy = y1.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3, f"max rel err {err.max():.3e}"


@pytest.mark.parametrize("M,K,N", FUSED)
def test_fused_default(M, K, N, monkeypatch):
    assert qoq.qoq_linear_workspace_bytes(M, N, K) == 0
    _check(M, K, N, monkeypatch)


@pytest.mark.parametrize("kw", [4, 8, 16])
def test_fused_every_wave_count(kw, monkeypatch):
    for (M, K, N) in FORCED:
        if K // 128 <= 4 * kw:
            _check(M, K, N, monkeypatch, cfg=f"fused,{kw}")


@pytest.mark.parametrize("kw", [4, 8, 16])
def test_fused_two_column_blocks_per_workgroup(kw, monkeypatch):
    """Workgroups of two 16-channel blocks (half as many workgroups repeat the
    token quantization), including a column count with an odd number of
    blocks (N = 400, 208: the last workgroup's second block lies past N)."""
    for (M, K, N) in FORCED:
        if K // 128 <= 4 * kw and not (kw == 16 and M > 12):
            _check(M, K, N, monkeypatch, cfg=f"fused,{kw},2")


def test_fused_configuration_out_of_lds_is_refused(monkeypatch):
    """16 waves of 16 token rows with two column blocks would need more than
    160 KiB of LDS: the plan refuses it (nothing launched)."""
    qoq.set_tuning("gemm", "fused,16,2")
    assert qoq.qoq_linear_path(13, 1040, 2048) == -1


@pytest.mark.parametrize("M,K,N", TWO_CALL)
def test_two_call_path(M, K, N, monkeypatch):
    assert qoq.qoq_linear_workspace_bytes(M, N, K) > 0
    _check(M, K, N, monkeypatch)


def test_forced_two_call_path_for_small_m(monkeypatch):
    _check(8, 1152, 400, monkeypatch, cfg="decode,1,1,8,4")


def test_zero_rows_and_empty_batch(monkeypatch):
    qoq.set_tuning("gemm", None)
    W, X, _ = wl.make_inputs(6, 1024, 96, seed=3)
    X[2] = 0
    X[5] = 0
    pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
    y, acc = qoq.w4a8_linear(_half(X), pw, acc_debug=True)
    ref = oracle.w4a8_linear(X, W)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    assert torch.all(y[2] == 0) and torch.all(y[5] == 0)
    y0 = qoq.w4a8_linear(torch.empty((0, 1024), dtype=torch.float16, device=DEV), pw)
    assert y0.shape == (0, 96)
