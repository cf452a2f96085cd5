"""Every compiled GEMM kernel configuration against the oracle.

The library picks a kernel family and tile per shape; QOQ_GEMM_CONFIG forces
one configuration (a name that is not compiled makes the call fail, so a
silently ignored override cannot pass). Each configuration must give the
oracle's INT32 accumulators bit-exactly on ragged shapes (odd group counts,
column counts that fill no tile, token counts that fill no tile) and the fp16
output within the relative tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

qoq = pytest.importorskip("bit_integer_gemm_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

DECODE = [(1, 1, 16, 2), (1, 1, 8, 2), (1, 2, 8, 2), (1, 2, 4, 2), (1, 4, 4, 2), (1, 4, 2, 2),
          (1, 8, 2, 2), (1, 1, 16, 4), (1, 2, 8, 4), (1, 4, 4, 4), (2, 1, 16, 2), (2, 1, 8, 2),
          (2, 2, 8, 2), (2, 2, 4, 2), (2, 4, 4, 2), (2, 4, 2, 2), (2, 8, 2, 2), (2, 2, 8, 4),
          (2, 4, 4, 4), (4, 1, 8, 2), (4, 2, 8, 2), (4, 2, 4, 2), (4, 4, 4, 2), (4, 4, 2, 2),
          (4, 4, 4, 4), (4, 1, 8, 4), (2, 1, 8, 4), (1, 1, 8, 4), (2, 1, 16, 4)]
LDS = [(1, 1, 4, 2), (1, 2, 4, 2), (1, 1, 8, 2), (1, 2, 8, 2), (1, 4, 4, 2), (2, 1, 4, 2),
       (2, 2, 4, 2), (2, 1, 8, 2), (2, 2, 8, 2), (2, 4, 4, 2), (4, 1, 4, 2), (4, 2, 4, 2),
       (4, 1, 8, 2), (4, 2, 8, 2), (4, 4, 4, 2), (4, 1, 4, 4), (4, 2, 4, 4), (4, 1, 8, 4),
       (4, 2, 8, 4), (8, 2, 4, 2), (8, 4, 4, 2), (16, 2, 4, 2), (16, 4, 4, 2), (8, 2, 8, 2),
       (4, 1, 6, 4), (4, 2, 6, 4), (4, 1, 12, 4), (4, 1, 12, 2), (4, 1, 16, 2), (1, 1, 6, 4),
       (1, 1, 12, 4), (2, 1, 6, 4), (2, 1, 12, 4), (4, 1, 12, 8), (4, 1, 8, 8), (4, 1, 6, 8),
       (4, 2, 6, 8), (4, 1, 4, 8)]
TILE32 = [(4, 2, 2, 2, 4), (4, 2, 1, 2, 4), (4, 1, 2, 2, 4), (2, 2, 2, 2, 4), (2, 1, 2, 2, 4),
          (8, 1, 1, 2, 4), (4, 2, 2, 1, 4), (8, 1, 2, 1, 4), (8, 2, 2, 1, 4), (2, 1, 2, 3, 4),
          (4, 1, 2, 3, 4), (2, 1, 4, 2, 4), (2, 1, 8, 2, 4), (2, 2, 4, 2, 4), (2, 1, 4, 3, 4),
          (2, 1, 8, 1, 4), (2, 2, 8, 1, 4), (4, 1, 4, 2, 4), (1, 1, 4, 3, 4), (1, 1, 2, 3, 4),
          (1, 1, 8, 2, 4), (1, 1, 4, 4, 4), (2, 1, 4, 1, 6), (2, 1, 2, 1, 6), (2, 1, 4, 1, 8),
          (2, 1, 2, 1, 8), (2, 1, 4, 1, 3), (2, 1, 4, 2, 3), (1, 1, 4, 1, 6), (2, 1, 8, 1, 6),
          (4, 1, 2, 1, 8), (4, 2, 2, 1, 8)]
GENERIC = [(1, 2), (2, 2), (4, 2)]

# (M, K, N): odd group counts, N not a multiple of any tile width
SHAPES_SMALL_M = [(1, 640, 208), (13, 1152, 400), (37, 384, 48), (64, 2048, 528)]
SHAPES_LARGE_M = [(100, 640, 208), (300, 1152, 528), (257, 256, 1040)]

_cases = {}


def _case(M, K, N):
    key = (M, K, N)
    if key not in _cases:
        W, X, _ = wl.make_inputs(M, K, N, seed=M + 3 * K + 7 * N)
        pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
        x8, s_x = qoq.quantize_act(torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV))
        ref = oracle.w4a8_linear(X, W)
        _cases[key] = (pw, x8, s_x, ref)
    return _cases[key]


def _run(monkeypatch, cfg, M, K, N):
    pw, x8, s_x, ref = _case(M, K, N)
    monkeypatch.setenv("QOQ_GEMM_CONFIG", cfg)
    print(f"\n[gpu-case] {cfg} M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    torch.cuda.synchronize()
    got = acc.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, ref["acc"]), f"{cfg}: acc differs at {np.argwhere(got != ref['acc'])[:4]}"
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3, f"{cfg}: max rel err {err.max():.3e}"


def _fmt(fam, cfg):
    return fam + "," + ",".join(str(v) for v in cfg)


@pytest.mark.parametrize("cfg", DECODE, ids=[_fmt("decode", c) for c in DECODE])
def test_decode_family(monkeypatch, cfg):
    for (M, K, N) in SHAPES_SMALL_M:
        if M <= 16 * cfg[0]:
            _run(monkeypatch, _fmt("decode", cfg), M, K, N)


SPLIT = [c for c in DECODE if c[0] < 4]


@pytest.mark.parametrize("cfg", SPLIT, ids=[_fmt("decode", c) for c in SPLIT])
def test_decode_family_row_tiles(monkeypatch, cfg):
    """More tokens than one workgroup's rows: 2 to 4 row tiles per column
    range (the last one ragged), paired 8 workgroup ids apart."""
    N = 16 * cfg[1] * 8 * 3
    for M in (40, 64):
        if M > 16 * cfg[0]:
            _run(monkeypatch, _fmt("decode", cfg), M, 1152, N)


@pytest.mark.parametrize("M,K,N", [(200, 1152, 512), (65, 256, 512), (256, 4096, 256), (129, 640, 4096)])
def test_decode_plan_for_a_few_hundred_tokens(M, K, N, monkeypatch):
    """Short, narrow layers at 65-256 tokens take the decode family by
    default (64-row tiles paired 8 workgroup ids apart), including fewer
    groups than waves."""
    monkeypatch.delenv("QOQ_GEMM_CONFIG", raising=False)
    pw, x8, s_x, ref = _case(M, K, N)
    print(f"\n[gpu-case] default plan M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3


@pytest.mark.parametrize("M,K,N", [(200, 256, 24576), (256, 384, 28672)])
def test_wide_layer_plan_for_a_few_hundred_tokens(M, K, N, monkeypatch):
    """Wide layers at 129-256 tokens with at least 192 tiles of 128 x 256
    take those tiles with 8 waves by default (the last row tile ragged for
    M = 200)."""
    monkeypatch.delenv("QOQ_GEMM_CONFIG", raising=False)
    pw, x8, s_x, ref = _case(M, K, N)
    print(f"\n[gpu-case] default plan M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3


def test_decode_row_tiles_need_whole_rounds(monkeypatch):
    """Row tiles pair workgroups 8 ids apart, which needs the column tiles in
    whole rounds of 8: otherwise the configuration is refused."""
    pw, x8, s_x, _ = _case(*SHAPES_SMALL_M[2])          # M = 37, N = 48: 3 column tiles
    monkeypatch.setenv("QOQ_GEMM_CONFIG", "decode,1,1,8,4")
    with pytest.raises(qoq.QoQError) as e:
        qoq.w4a8_gemm(x8, s_x, pw)
    assert e.value.status == 8


@pytest.mark.parametrize("cfg", LDS, ids=[_fmt("lds", c) for c in LDS])
def test_shared_activation_family(monkeypatch, cfg):
    for (M, K, N) in SHAPES_SMALL_M + SHAPES_LARGE_M[:1]:
        _run(monkeypatch, _fmt("lds", cfg), M, K, N)


# split K: (family, config, requested splits); with K = 2560 (20 groups) a
# request of 2 gives ranges of 16 + 4 groups, 3 or more gives 8 + 8 + 4;
# K = 1152 gives 8 + 1; K = 640 (5 groups) stays one range
SPLITK = [("lds", (4, 1, 4, 2), 2), ("lds", (4, 1, 4, 2), 3), ("lds", (4, 1, 8, 4), 4),
          ("lds", (2, 1, 8, 2), 64), ("lds", (1, 1, 4, 2), 2), ("lds", (4, 2, 4, 2), 3),
          ("lds", (4, 1, 12, 8), 2), ("lds", (4, 1, 16, 2), 2), ("tile32", (2, 1, 2, 2, 4), 3), ("tile32", (2, 1, 4, 1, 8), 2),
          ("tile32", (4, 1, 2, 1, 8), 4), ("tile32", (1, 1, 4, 3, 4), 64),
          ("tile32", (2, 2, 2, 2, 4), 2), ("tile32", (2, 1, 8, 2, 4), 3)]
SPLITK_SHAPES = [(1, 2560, 208), (37, 1152, 400), (64, 2560, 528), (50, 3072, 1040), (13, 640, 208),
                 (100, 2560, 208)]


@pytest.mark.parametrize("fam,cfg,splits", SPLITK, ids=[_fmt(f, c) + f",{s}" for f, c, s in SPLITK])
def test_split_k(monkeypatch, fam, cfg, splits):
    """K split over workgroups: exact INT32 partials in the workspace, added
    by a second kernel that applies the epilogue."""
    name = _fmt(fam, cfg) + f",{splits}"
    for (M, K, N) in SPLITK_SHAPES:
        monkeypatch.setenv("QOQ_GEMM_CONFIG", name)
        ng = K // 128
        gps = min(ng, -(-(-(-ng // splits)) // 8) * 8)
        nsplit = -(-ng // gps)
        want = nsplit * M * N * 4 if nsplit > 1 else 0
        assert qoq.qoq_gemm_workspace_bytes(M, N, K) == want
        _run(monkeypatch, name, M, K, N)


def test_split_k_needs_its_workspace(monkeypatch):
    pw, x8, s_x, _ = _case(64, 2560, 528)
    monkeypatch.setenv("QOQ_GEMM_CONFIG", "lds,4,1,4,2,3")
    need = qoq.qoq_gemm_workspace_bytes(64, 528, 2560)
    assert need == 3 * 64 * 528 * 4
    y = torch.empty((64, 528), dtype=torch.float16, device=DEV)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    st = qoq.qoq_w4a8_gemm(x8.data_ptr(), s_x.data_ptr(), 64, 2560, pw.packed.data_ptr(),
                           pw.s1.data_ptr(), 528, 128, y.data_ptr(), None, ws.data_ptr(), need - 1,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 5                                          # QOQ_ERR_WORKSPACE
    st = qoq.qoq_w4a8_gemm(x8.data_ptr(), s_x.data_ptr(), 64, 2560, pw.packed.data_ptr(),
                           pw.s1.data_ptr(), 528, 128, y.data_ptr(), None, None, 0,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 5


@pytest.mark.parametrize("cfg", TILE32, ids=[_fmt("tile32", c) for c in TILE32])
def test_tile32_family(monkeypatch, cfg):
    for (M, K, N) in SHAPES_LARGE_M + SHAPES_SMALL_M[1:2]:
        _run(monkeypatch, _fmt("tile32", cfg), M, K, N)


@pytest.mark.parametrize("cfg", GENERIC, ids=[_fmt("generic", c) for c in GENERIC])
def test_generic_family(monkeypatch, cfg):
    for (M, K, N) in SHAPES_SMALL_M[:2] + SHAPES_LARGE_M[:1]:
        _run(monkeypatch, _fmt("generic", cfg), M, K, N)


def test_unknown_configuration_is_an_error(monkeypatch):
    pw, x8, s_x, _ = _case(*SHAPES_SMALL_M[0])
    for bad in ("tile32,99,1,1,1", "decode,1,3,3,3", "nonsense"):
        monkeypatch.setenv("QOQ_GEMM_CONFIG", bad)
        with pytest.raises(qoq.QoQError) as e:
            qoq.w4a8_gemm(x8, s_x, pw)
        assert e.value.status == 8
