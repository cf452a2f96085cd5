"""Every compiled GEMM kernel configuration against the oracle.

The library picks a kernel family and tile per shape; the "gemm" tuning override forces
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
from guard import Guarded, GuardedWorkspace

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

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
STREAM = [(2, 1, 8, 4, 8), (2, 1, 8, 4, 4), (2, 1, 6, 4, 8), (2, 1, 4, 4, 8), (2, 1, 8, 8, 8),
          (2, 2, 8, 4, 8), (2, 1, 12, 4, 8), (1, 1, 8, 4, 8), (1, 2, 8, 4, 8), (2, 1, 16, 4, 8),
          (2, 1, 3, 4, 8), (1, 1, 4, 4, 8), (2, 2, 4, 4, 8), (2, 1, 6, 8, 8)]
WIDE = [(4, 2, 8, 3, 1), (4, 2, 8, 4, 1), (8, 1, 8, 3, 1), (8, 1, 8, 4, 1), (4, 1, 8, 4, 1),
        (4, 2, 4, 4, 1), (4, 1, 4, 4, 2), (2, 1, 8, 4, 1), (8, 2, 4, 3, 1), (8, 2, 4, 4, 1)]
KSPLIT = [(1, 1, 8, 2), (1, 2, 8, 2), (2, 1, 8, 2), (2, 2, 8, 2), (4, 1, 8, 2), (2, 2, 4, 2),
          (4, 1, 4, 2), (2, 1, 8, 4), (1, 1, 16, 2), (2, 3, 4, 2), (1, 3, 8, 2), (2, 2, 4, 3),
          (2, 2, 4, 4), (2, 3, 4, 3), (2, 3, 4, 4), (4, 1, 4, 3), (4, 1, 4, 4), (1, 1, 8, 4),
          (1, 2, 8, 3), (2, 1, 8, 3)]

# (M, K, N): odd group counts, N not a multiple of any tile width
SHAPES_SMALL_M = [(1, 640, 208), (13, 1152, 400), (37, 384, 48), (64, 2048, 528)]
SHAPES_LARGE_M = [(100, 640, 208), (300, 1152, 528), (257, 256, 1040)]

_cases = {}


def _case(M, K, N):
    """Packed weights, quantized activations (written inside guard bands) and
    the oracle's result for one seeded shape."""
    key = (M, K, N)
    if key not in _cases:
        W, X, _ = wl.make_inputs(M, K, N, seed=M + 3 * K + 7 * N)
        pw = qoq.pack_weights(torch.from_numpy(W).to(DEV))
        gx8 = Guarded(((M + 15) // 16, K // 16, 16, 16), torch.int8, DEV)
        gsx = Guarded((M,), torch.float32, DEV)
        x8, s_x = qoq.quantize_act(torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(DEV),
                                   out=(gx8.t, gsx.t))
        gx8.check("x8")
        gsx.check("s_x")
        ref = oracle.w4a8_linear(X, W)
        _cases[key] = (pw, x8, s_x, ref)
    return _cases[key]


def _run(monkeypatch, cfg, M, K, N):
    """One forced configuration: accumulators bit-exact, y within the
    tolerance, and nothing written outside y, the accumulators or the
    workspace (guard bands on all three)."""
    pw, x8, s_x, ref = _case(M, K, N)
    qoq.set_tuning("gemm", cfg)
    print(f"\n[gpu-case] {cfg} M={M} K={K} N={N}", flush=True)
    gy = Guarded((M, N), torch.float16, DEV)
    gacc = Guarded((M, N), torch.int32, DEV)
    ws = GuardedWorkspace(qoq.qoq_gemm_workspace_bytes(M, N, K), DEV)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=gacc.t, y=gy.t, workspace=ws)
    torch.cuda.synchronize()
    gy.check("y")
    gacc.check("acc_debug")
    ws.check()
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


def _default_plan(M, K, N):
    """The default plan for a shape: accumulators bit-exact, y within the
    tolerance."""
    qoq.set_tuning("gemm", None)
    pw, x8, s_x, ref = _case(M, K, N)
    print(f"\n[gpu-case] default plan M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3


@pytest.mark.parametrize("M,K,N", [(16, 1024, 8192), (5, 2048, 8192), (16, 1024, 32768),
                                   (3, 1024, 33024), (12, 8192, 18432)])
def test_plans_for_up_to_16_tokens_on_wide_layers(M, K, N, monkeypatch):
    """Up to 16 tokens: the decode family with two 16-column blocks per
    workgroup on 512-block layers (N = 8192), the shared-activation family
    with two blocks per wave on layers of 2048 blocks or more (N = 33024: an
    odd block count, the last wave's second block outside), and for 9-16
    tokens on 18432-30720-column layers with K >= 8192 the K-split family's
    32 x 96 tiles."""
    _default_plan(M, K, N)


@pytest.mark.parametrize("M,K,N", [(65, 256, 512), (128, 1152, 4096), (100, 4096, 256),
                                   (96, 4096, 6144)])
def test_ksplit_plan_for_65_to_128_tokens(M, K, N, monkeypatch):
    """Narrow layers with short K (at most 32 groups) at 65-128 tokens take
    the K-split 32x32 family's 64 x 64 tiles by default, including fewer
    groups than waves and a ragged second row tile."""
    qoq.set_tuning("gemm", None)
    pw, x8, s_x, ref = _case(M, K, N)
    print(f"\n[gpu-case] default plan M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3


@pytest.mark.parametrize("M,K,N", [(200, 1152, 512), (256, 4096, 256), (129, 640, 4096),
                                   (256, 640, 6144), (193, 1920, 8192), (256, 384, 2064)])
def test_ksplit_plan_for_a_few_hundred_tokens(M, K, N, monkeypatch):
    """Narrow layers (N <= 8192) at 129-256 tokens take the K-split 32x32
    family by default: 64-row tiles of 64 columns, or of 96 columns when
    that is closer to one workgroup per CU (N = 6144, 8192); ragged rows
    (M = 129, 193, 200), fewer groups than waves (K = 256 / 384), odd
    column counts (N = 2064: the last 32-column tile half outside)."""
    qoq.set_tuning("gemm", None)
    pw, x8, s_x, ref = _case(M, K, N)
    print(f"\n[gpu-case] default plan M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3


@pytest.mark.parametrize("M,K,N", [(40, 8192, 18432), (48, 4096, 18432)])
def test_ksplit_plan_for_wide_layers_at_64_tokens(M, K, N, monkeypatch):
    """33-64 tokens on layers of 18432-30720 columns take the K-split
    family's 64 x 96 tiles by default when K >= 8192 (M = 40: rows 40-63 of
    the tile padded), the shared-activation family when K = 4096."""
    qoq.set_tuning("gemm", None)
    pw, x8, s_x, ref = _case(M, K, N)
    print(f"\n[gpu-case] default plan M={M} K={K} N={N}", flush=True)
    y, acc = qoq.w4a8_gemm(x8, s_x, pw, acc_debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    yy = y.cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref["y"]) / np.maximum(np.abs(ref["y"]), 2.0 ** -14)
    assert err.max() <= 2e-3


@pytest.mark.parametrize("M,K,N", [(192, 256, 36864), (200, 256, 36864), (512, 256, 32768)])
def test_wide_tile_plan_when_tiles_fill_rounds(M, K, N, monkeypatch):
    """Past 128 tokens, shapes whose 256 x 256 tiles need no more rounds of
    the CUs than twice the 128 x 256 tiles' (and pad the rows no further)
    take the wide-tile family by default: 144 tiles at M = 192 and 200 (rows
    padded to 256), 256 tiles at M = 512."""
    qoq.set_tuning("gemm", None)
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
    qoq.set_tuning("gemm", None)
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
    qoq.set_tuning("gemm", "decode,1,1,8,4")
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
        qoq.set_tuning("gemm", name)
        ng = K // 128
        gps = min(ng, -(-(-(-ng // splits)) // 8) * 8)
        nsplit = -(-ng // gps)
        want = nsplit * M * N * 4 if nsplit > 1 else 0
        assert qoq.qoq_gemm_workspace_bytes(M, N, K) == want
        _run(monkeypatch, name, M, K, N)


@pytest.mark.parametrize("K", [10240, 17408])
def test_split_k_more_than_eight_partials(monkeypatch, K):
    """The second kernel adds the partials in batches of 8: 10 and 17 of them
    (8-group splits of 80 and 136 groups) take two and three batches, the
    last one short."""
    name = "lds,2,1,8,2,64"
    qoq.set_tuning("gemm", name)
    assert qoq.qoq_gemm_workspace_bytes(37, 208, K) == (K // 1024) * 37 * 208 * 4
    _run(monkeypatch, name, 37, K, 208)


def test_split_k_needs_its_workspace(monkeypatch):
    pw, x8, s_x, _ = _case(64, 2560, 528)
    qoq.set_tuning("gemm", "lds,4,1,4,2,3")
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
        qoq.set_tuning("gemm", bad)
        with pytest.raises(qoq.QoQError) as e:
            qoq.w4a8_gemm(x8, s_x, pw)
        assert e.value.status == 8


@pytest.mark.parametrize("cfg", KSPLIT, ids=[_fmt("ksplit", c) for c in KSPLIT])
def test_ksplit32_family(monkeypatch, cfg):
    for (M, K, N) in SHAPES_SMALL_M + SHAPES_LARGE_M:
        _run(monkeypatch, _fmt("ksplit", cfg), M, K, N)


# The K-split kernel reads a wave's group records into LDS once when the
# wave's K range has at most 57 groups (8 chunks of 8 groups, the range
# starting anywhere in its first chunk) and per group otherwise. Random
# weights (every group its own record) on both sides of that limit, with
# the waves' ranges starting at every offset inside a chunk (57 w mod 8 for
# w = 0..7: 0, 1, ..., 7).
KSPLIT_RECORD_LIMIT = [((2, 2, 4, 3), 4 * 57 * 128), ((2, 2, 4, 3), 4 * 58 * 128),
                       ((2, 1, 8, 2), 8 * 57 * 128), ((2, 1, 8, 2), 8 * 58 * 128),
                       ((1, 3, 8, 2), 8 * 57 * 128)]


@pytest.mark.parametrize("cfg,K", KSPLIT_RECORD_LIMIT,
                         ids=[f"{_fmt('ksplit', c)}@K{k}" for c, k in KSPLIT_RECORD_LIMIT])
def test_ksplit32_records_at_the_staging_limit(monkeypatch, cfg, K):
    _run(monkeypatch, _fmt("ksplit", cfg), 37, K, 208)


@pytest.mark.parametrize("cfg", WIDE, ids=[_fmt("wide", c) for c in WIDE])
def test_wide_family(monkeypatch, cfg):
    for (M, K, N) in SHAPES_LARGE_M + SHAPES_SMALL_M[1:2]:
        _run(monkeypatch, _fmt("wide", cfg), M, K, N)


@pytest.mark.parametrize("cfg,splits", [((4, 2, 8, 4, 1), 2), ((8, 1, 8, 3, 1), 3)],
                         ids=["wide,4,2,8,4,1/2", "wide,8,1,8,3,1/3"])
def test_wide_family_split_k(monkeypatch, cfg, splits):
    """K in whole chunks of 8 groups per workgroup row, partial sums added by
    the second kernel: 2560 inputs = 20 groups in ranges of 16 + 4 (two
    splits) or 8 + 8 + 4 (three)."""
    for (M, K, N) in [(300, 2560, 528), (64, 2560, 1040)]:
        _run(monkeypatch, _fmt("wide", cfg) + f",{splits}", M, K, N)


@pytest.mark.parametrize("cfg", STREAM, ids=[_fmt("stream", c) for c in STREAM])
def test_stream_family(monkeypatch, cfg):
    for (M, K, N) in SHAPES_SMALL_M + SHAPES_LARGE_M[:1]:
        _run(monkeypatch, _fmt("stream", cfg), M, K, N)


@pytest.mark.parametrize("cfg,splits", [((2, 1, 8, 4, 8), 2), ((2, 1, 4, 4, 8), 3), ((1, 1, 8, 4, 8), 4)],
                         ids=["stream,2,1,8,4,8/2", "stream,2,1,4,4,8/3", "stream,1,1,8,4,8/4"])
def test_stream_family_split_k(monkeypatch, cfg, splits):
    """K ranges of whole 8-group record chunks per workgroup row (20 groups:
    16 + 4, 8 + 8 + 4, or 8 + 8 + 4 with an empty fourth range folded away),
    chunks of activations shorter than CH at the end of a range."""
    for (M, K, N) in [(64, 2560, 528), (17, 2560, 1040), (100, 2560, 208)]:
        _run(monkeypatch, _fmt("stream", cfg) + f",{splits}", M, K, N)
