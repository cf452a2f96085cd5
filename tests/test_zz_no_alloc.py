"""The allocation-free GEMM entry point (qoq_w4a8_gemm_noalloc) against
qoq_w4a8_gemm with a caller workspace.

Both run the same kernels; the no-alloc call keeps split-K partial sums in
the library's fixed per-GPU scratch array instead of the workspace. Two calls
in a row on one GPU, the second with a smaller input, so the second reads a
scratch array that still holds the first call's partial sums: outputs and
INT32 accumulators must equal the workspace path's bit for bit (and the
accumulators the oracle's).
"""
import ctypes

import numpy as np
import pytest
import torch

import bit_integer_gemm_amd as qoq
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (first call, second smaller call): K split over workgroups in the default
# plan of every shape (shared-activation and 32x32-tile families), plus a
# shape with no split (scratch unused) between split ones
PAIRS = [((64, 16384, 4096), (40, 16384, 4096)),
         ((128, 8192, 1024), (96, 8192, 1024)),
         ((64, 16384, 4096), (8, 1024, 512))]


def _inputs(M, K, N):
    W, X, _ = wl.make_inputs(M, K, N, seed=11 * M + K + 3 * N)
    pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
    x8, s_x = qoq.quantize_act(torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV))
    return W, X, pw, x8, s_x


def _noalloc(x8, s_x, pw, M):
    y = torch.empty((M, pw.N), dtype=torch.float16, device=DEV)
    acc = torch.empty((M, pw.N), dtype=torch.int32, device=DEV)
    st = qoq.qoq_w4a8_gemm_noalloc(x8.data_ptr(), s_x.data_ptr(), M, pw.K, pw.packed.data_ptr(),
                                   pw.s1.data_ptr(), pw.N, 128, y.data_ptr(), acc.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, qoq.qoq_status_string(st)
    return y, acc


@pytest.mark.parametrize("pair", PAIRS, ids=[f"{a}->{b}" for a, b in PAIRS])
def test_noalloc_matches_workspace_path(pair):
    for (M, K, N) in pair:
        print(f"\n[gpu-case] noalloc M={M} K={K} N={N} "
              f"ws={qoq.qoq_gemm_workspace_bytes(M, N, K)}", flush=True)
        W, X, pw, x8, s_x = _inputs(M, K, N)
        y0, acc0 = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True, workspace=qoq.Workspace(DEV))
        y1, acc1 = _noalloc(x8, s_x, pw, M)
        torch.cuda.synchronize()
        assert torch.equal(acc0, acc1)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        if M * K * N <= 64 * 16384 * 4096:
            ref = oracle.w4a8_linear(X, W)
            assert np.array_equal(acc1.cpu().numpy().astype(np.int64), ref["acc"])


def test_noalloc_refuses_oversized_split():
    """A shape whose split-K partial sums exceed the scratch array is
    refused before anything is launched (no buffer is touched)."""
    M, K, N = 1280, 24576, 8192
    assert qoq.qoq_gemm_workspace_bytes(M, N, K) > qoq.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: the call refuses first
    st = qoq.qoq_w4a8_gemm_noalloc(fake, fake, M, K, fake, fake, N, 128, fake, None, None)
    assert qoq.QOQ_STATUS[st] == "QOQ_ERR_WORKSPACE"
