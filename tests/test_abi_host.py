"""The C-ABI library on the host (no GPU): it loads, exports every entry
point its header declares, sizes buffers, and rejects invalid arguments with
the documented status before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qoq.h")

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

OK, NULL, SHAPE, ALIGN, GROUP, WORKSPACE, HIP, FLAGS = range(8)
P = 0x10000  # a 16-byte aligned address that is never dereferenced


def header_functions():
    text = "".join(open(os.path.join(ROOT, "include", f)).read()
                   for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qoq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = qoq.lib()
    names = header_functions()
    assert set(names) >= {"qoq_pack_weights", "qoq_quantize_act", "qoq_w4a8_gemm",
                          "qoq_packed_weight_bytes", "qoq_gemm_workspace_bytes",
                          "qoq_act_bytes", "qoq_status_string", "qoq_w4a8_linear",
                          "qoq_linear_workspace_bytes"}
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_variant_sizes_and_validation(monkeypatch):
    qoq.set_tuning("variant", None)
    L = qoq.lib()
    assert L.qoq_w8a8_weight_bytes(4096, 4096) == 4096 * 4096
    assert L.qoq_w8a8_weight_bytes(4008, 4096) == 0
    assert L.qoq_w4a4_weight_bytes(4096, 4096) == qoq.qoq_packed_weight_bytes(4096, 4096)
    # x4 codes (rows padded to 16, K/2 bytes each), then fp32 scales [K/128][M padded to 128]
    assert L.qoq_w4a4_act_bytes(1, 4096) == 16 * 2048 + 32 * 128 * 4
    assert L.qoq_w4a4_act_bytes(200, 256) == 208 * 128 + 2 * 256 * 4
    assert L.qoq_w4a4_act_bytes(0, 4096) == 0 and L.qoq_w4a4_act_bytes(4, 100) == 0
    assert L.qoq_w8a8_gemm(P, P, 4, 4000, P, P, 4096, P, None, None) == SHAPE
    assert L.qoq_w8a8_gemm(None, P, 4, 4096, P, P, 4096, P, None, None) == NULL
    assert L.qoq_w8a8_gemm(P + 1, P, 4, 4096, P, P, 4096, P, None, None) == ALIGN
    assert L.qoq_w8a8_gemm(P, P, 0, 4096, P, P, 4096, P, None, None) == OK
    assert L.qoq_w4a4_gemm(P, 4, 4096, P, 4008, P, None) == SHAPE
    assert L.qoq_w4a4_gemm(P, 4, 4096, None, 4096, P, None) == NULL
    assert L.qoq_w4a4_quantize_act(P, 4, 200, P, None) == SHAPE
    assert L.qoq_w4a4_quantize_act(P + 2, 4, 256, P, None) == ALIGN
    # W4A16: nibbles, then the scale records, then the zero records
    assert L.qoq_w4a16_weight_bytes(4096, 4096) == 4096 * 2048 + 2 * (4096 // 16) * 4 * 256
    assert L.qoq_w4a16_weight_bytes(16, 640) == 16 * 320 + 2 * 256
    assert L.qoq_w4a16_weight_bytes(4008, 4096) == 0 and L.qoq_w4a16_weight_bytes(16, 100) == 0
    assert L.qoq_w4a16_pack_weights(None, 16, 128, P, None) == NULL
    assert L.qoq_w4a16_pack_weights(P, 16, 120, P, None) == SHAPE
    assert L.qoq_w4a16_gemm(P, 4, 4096, P, 4008, P, None) == SHAPE
    assert L.qoq_w4a16_gemm(P, -1, 4096, P, 4096, P, None) == SHAPE
    assert L.qoq_w4a16_gemm(P, 4, 4096, P, 4096, None, None) == NULL
    assert L.qoq_w4a16_gemm(P + 2, 4, 4096, P, 4096, P, None) == ALIGN
    assert L.qoq_w4a16_gemm(P, 0, 4096, P, 4096, P, None) == OK
    assert L.qoq_w4a16_gemm(P, 1 << 20, 1024, P, 4096, P, None) == SHAPE   # 2 M K = 2^31
    # the comparison kernels address with 32-bit buffer offsets: weights of
    # 2^31 bytes or more are refused before any launch
    assert L.qoq_w8a8_gemm(P, P, 4, 1 << 16, P, P, 1 << 15, P, None, None) == SHAPE   # N K = 2^31
    assert L.qoq_w4a4_gemm(P, 4, 1 << 17, P, 1 << 15, P, None) == SHAPE             # N K / 2 = 2^31
    assert L.qoq_w4a16_gemm(P, 4, 1 << 17, P, 1 << 15, P, None) == SHAPE
    qoq.set_tuning("variant", "9,9,9,9,9")
    assert L.qoq_w8a8_gemm(P, P, 4, 4096, P, P, 4096, P, None, None) == 8
    assert L.qoq_w4a4_gemm(P, 4, 4096, P, 4096, P, None) == 8
    assert L.qoq_w4a16_gemm(P, 4, 4096, P, 4096, P, None) == 8


def test_kv4_sizes_and_validation(monkeypatch):
    qoq.set_tuning("kv4_splits", None)
    L = qoq.lib()
    assert L.qoq_kv4_cache_bytes(64, 8, 2048, 128) == 64 * 8 * 2048 * 133
    assert L.qoq_kv4_cache_bytes(2, 8, 100, 128) == 0          # capacity not a multiple of 32
    assert L.qoq_kv4_cache_bytes(2, 8, 64, 64) == 0            # head dim other than 128
    assert L.qoq_kv4_cache_bytes(0, 8, 64, 128) == 0
    assert L.qoq_kv4_cache_bytes(1 << 30, 4096, 1 << 24, 128) == 0     # offsets beyond int64
    assert L.qoq_kv16_cache_bytes(64, 8, 2048, 128) == 64 * 8 * 2048 * 512
    # one workgroup per (sequence, KV head) when there are 512 of them: no
    # workspace; few long contexts are split (here 16 ways) and their partial
    # results (132 floats per query head and split) meet in the workspace
    assert L.qoq_kv4_attention_workspace_bytes(64, 32, 8, 128, 2048) == 0
    assert L.qoq_kv4_attention_workspace_bytes(4, 32, 8, 128, 16384) == 4 * 32 * 16 * 132 * 4
    qoq.set_tuning("kv4_splits", "3")
    assert L.qoq_kv4_attention_workspace_bytes(4, 32, 8, 128, 16384) == 4 * 32 * 3 * 132 * 4
    qoq.set_tuning("kv4_splits", None)
    att = L.qoq_kv4_decode_attention
    assert att(P, 2, 32, 8, 64, P, P, 64, P, 64, P, None, 0, None) == SHAPE      # D
    assert att(P, 2, 30, 8, 128, P, P, 64, P, 64, P, None, 0, None) == SHAPE     # H % H_kv
    assert att(P, 2, 64, 2, 128, P, P, 64, P, 64, P, None, 0, None) == SHAPE     # group of 32
    assert att(P, 2, 32, 8, 128, P, P, 64, P, 65, P, None, 0, None) == SHAPE     # max_len > capacity
    assert att(P, 2, 32, 8, 128, P, P, 60, P, 32, P, None, 0, None) == SHAPE     # capacity % 32
    assert att(P, 0, 32, 8, 128, None, None, 64, None, 64, None, None, 0, None) == OK
    assert att(None, 2, 32, 8, 128, P, P, 64, P, 64, P, None, 0, None) == NULL
    assert att(P, 2, 32, 8, 128, P, P, 64, None, 64, P, None, 0, None) == NULL
    assert att(P + 2, 2, 32, 8, 128, P, P, 64, P, 64, P, None, 0, None) == ALIGN
    assert att(P, 4, 32, 8, 128, P, P, 16384, P, 16384, P, None, 0, None) == WORKSPACE
    assert att(P, 4, 32, 8, 128, P, P, 16384, P, 16384, P, P, 1024, None) == WORKSPACE
    # a dispatch counts its work-items in 32 bits: 2^20 sequences x 64 query
    # heads (64 work-items each in the merge, 2^32 in all) are refused, and
    # have no workspace size
    assert att(P, 1 << 20, 64, 64, 128, P, P, 32, P, 32, P, None, 0, None) == SHAPE
    assert L.qoq_kv16_decode_attention(P, 1 << 20, 64, 64, 128, P, 32, P, 32, P, None, 0,
                                       None) == SHAPE
    assert L.qoq_kv4_attention_workspace_bytes(1 << 20, 64, 64, 128, 32) == 0
    qoq.set_tuning("kv4_splits", "1000000000")   # clamped to 2^16 splits
    assert att(P, 64, 32, 8, 128, P, P, 1 << 20, P, 1 << 20, P, None, 0, None) == SHAPE
    qoq.set_tuning("kv4_splits", None)
    app = L.qoq_kv4_append
    assert app(P, P, 2, 0, 8, 128, P, P, P, 64, None) == OK
    assert app(P, P, 2, 5, 8, 128, P, None, P, 64, None) == NULL
    assert app(P, P + 4, 2, 5, 8, 128, P, P, P, 64, None) == ALIGN
    assert app(P, P, 2, 5, 8, 100, P, P, P, 64, None) == SHAPE
    assert app(P, P, 2, 5, 8, 128, P, P, P, 48, None) == SHAPE
    sm = L.qoq_kv4_smooth_factors
    assert sm(P, 0, 8, 128, P, None) == SHAPE
    assert sm(None, 4, 8, 128, P, None) == NULL
    assert sm(P, 4, 8, 128, P + 2, None) == ALIGN


def test_status_strings():
    for s in range(8):
        assert qoq.qoq_status_string(s)
    assert qoq.qoq_status_string(99) == "unknown status"


def test_packed_weight_bytes():
    # nibbles N*K/2 + records NB * ceil(NG/8) * 256
    assert qoq.qoq_packed_weight_bytes(4096, 4096) == 4096 * 4096 // 2 + 256 * 4 * 256
    assert qoq.qoq_packed_weight_bytes(16, 128) == 1024 + 256
    assert qoq.qoq_packed_weight_bytes(16, 1152) == 9 * 1024 + 2 * 256
    for bad in [(0, 128), (16, 0), (8, 128), (16, 64), (-16, 128), (16, 200)]:
        assert qoq.qoq_packed_weight_bytes(*bad) == 0
    assert qoq.qoq_packed_weight_bytes(16, 128, 64) == 0


def test_act_bytes():
    # rows padded to tiles of 16, K bytes per row
    assert qoq.qoq_act_bytes(1, 4096) == 16 * 4096
    assert qoq.qoq_act_bytes(16, 128) == 16 * 128
    assert qoq.qoq_act_bytes(17, 256) == 32 * 256
    assert qoq.qoq_act_bytes(4096, 4096) == 4096 * 4096
    for bad in [(0, 128), (-1, 128), (4, 0), (4, 100), (4, -128)]:
        assert qoq.qoq_act_bytes(*bad) == 0


def test_act_layout_formula_is_a_bijection():
    # the documented tile layout maps the M x K codes one-to-one into the
    # first 16*ceil(M/16)*K bytes, and act_rows inverts it
    from act_layout import act_offset, act_rows
    M, K = 37, 384
    size = qoq.qoq_act_bytes(M, K)
    m, k = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    off = act_offset(m, k, K)
    assert off.min() >= 0 and off.max() < size
    assert len(np.unique(off)) == M * K
    codes = np.arange(M * K, dtype=np.int64).reshape(M, K)
    buf = np.full(size, -1, np.int64)
    buf[off.ravel()] = codes.ravel()
    assert np.array_equal(act_rows(buf.reshape(-1, K // 16, 16, 16), M), codes)


def test_workspace_bytes():
    assert qoq.qoq_gemm_workspace_bytes(0, 4096, 4096) == 0
    assert qoq.qoq_gemm_workspace_bytes(1, 10, 4096) == 0
    for M in (1, 8, 32, 64):
        ws = qoq.qoq_gemm_workspace_bytes(M, 4096, 4096)
        if ws:
            assert ws >= M * 4096 * 4 and ws % 256 == 0


def test_split_k_workspace_bytes(monkeypatch):
    """The shared-activation family split over K keeps INT32 partial sums
    [splits][M][N] in the workspace; ranges are whole chunks of 8 groups."""
    for cfg, M, N, K, splits in [("lds,4,1,4,2,3", 64, 528, 2560, 3),     # 8 + 8 + 4 groups
                                 ("lds,4,1,4,2,2", 64, 528, 2560, 2),     # 16 + 4
                                 ("lds,4,1,4,2,64", 50, 1040, 3072, 3),   # 8 + 8 + 8
                                 ("lds,4,1,4,2,4", 64, 528, 640, 1),      # 5 groups: one range
                                 ("lds,4,1,4,2,1", 64, 528, 2560, 1),
                                 ("tile32,2,1,2,2,4,3", 64, 528, 2560, 3),
                                 ("tile32,4,1,2,1,8,2", 300, 1040, 1152, 2)]:   # 8 + 1
        qoq.set_tuning("gemm", cfg)
        want = splits * M * N * 4 if splits > 1 else 0
        assert qoq.qoq_gemm_workspace_bytes(M, N, K) == want, cfg
        # the two-call linear path carves the same partials after x8 and s_x
        act = -(-qoq.qoq_act_bytes(M, K) // 256) * 256 + -(-4 * M // 256) * 256
        assert qoq.qoq_linear_workspace_bytes(M, N, K) == act + want, cfg
    for bad in ("lds,4,1,4,2,0", "lds,4,1,4,2,65", "lds,4,3,4,2,2", "tile32,2,1,2,2,4,0",
                "tile32,2,1,2,2,4,65"):
        qoq.set_tuning("gemm", bad)
        assert qoq.qoq_gemm_workspace_bytes(64, 528, 2560) == 0
        assert qoq.qoq_w4a8_gemm(P, P, 64, 2560, P, P, 528, 128, P, None, None, 0, None) == 8


def test_stream_read_rejects_bad_arguments():
    f = qoq.qoq_stream_read
    assert f(None, 1024, 0, P, None) == NULL
    assert f(P, 1024, 0, None, None) == NULL
    for nbytes, wg in [(0, 0), (1000, 0), (1024, -1), (1024, 65537), ((1 << 40) + 16, 0)]:
        assert f(P, nbytes, wg, P, None) == SHAPE, (nbytes, wg)
    assert f(P + 8, 1024, 0, P, None) == ALIGN


def test_default_plans_split_long_k(monkeypatch):
    """The planner splits K for long-K shapes over few output tiles (the
    workspace then holds splits x M x N INT32 partials) and nowhere else."""
    qoq.set_tuning("gemm", None)
    ws = qoq.qoq_gemm_workspace_bytes
    assert ws(64, 8192, 24576) == 4 * 64 * 8192 * 4          # Qwen1.5-72B down, M = 64
    assert ws(1024, 8192, 24576) == 2 * 1024 * 8192 * 4      # Qwen1.5-72B down, M = 1024
    for M, N, K in [(1, 4096, 4096), (8, 4096, 4096), (32, 4096, 4096), (64, 4096, 4096),
                    (64, 49152, 8192), (256, 6144, 4096), (256, 4096, 4096), (256, 28672, 4096),
                    (4096, 14336, 4096), (1024, 49152, 8192), (1024, 24576, 8192), (16, 512, 512),
                    (256, 4096, 14336), (64, 24576, 8192)]:
        assert ws(M, N, K) == 0, (M, N, K)


def test_pack_rejects_bad_arguments():
    f = qoq.qoq_pack_weights
    assert f(P, 4096, 4096, 64, P, P, None, 0, None) == GROUP
    assert f(P, 4096, 4000, 128, P, P, None, 0, None) == SHAPE
    assert f(P, 4090, 4096, 128, P, P, None, 0, None) == SHAPE
    assert f(P, -16, 4096, 128, P, P, None, 0, None) == SHAPE
    assert f(P, 16, 128, 128, P, P, None, 0x2, None) == FLAGS
    assert f(None, 16, 128, 128, P, P, None, 0, None) == NULL
    assert f(P, 16, 128, 128, None, P, None, 0, None) == NULL
    assert f(P, 16, 128, 128, P, None, None, 0, None) == NULL
    assert f(P + 4, 16, 128, 128, P, P, None, 0, None) == ALIGN
    assert f(P, 16, 128, 128, P + 8, P, None, 0, None) == ALIGN
    # canonical: input required with the flag, all three pointers or none
    assert f(None, 16, 128, 128, P, None, None, 1, None) == NULL
    assert f(None, 16, 128, 128, P, None, (P, 0, P), 1, None) == NULL
    assert f(P, 16, 128, 128, P, P, (P, P, 0), 0, None) == NULL


def test_quantize_act_rejects_bad_arguments():
    f = qoq.qoq_quantize_act
    assert f(P, -1, 128, P, P, None) == SHAPE
    assert f(P, 4, 100, P, P, None) == SHAPE
    assert f(P, 4, 0, P, P, None) == SHAPE
    assert f(None, 4, 128, P, P, None) == NULL
    assert f(P, 4, 128, None, P, None) == NULL
    assert f(P, 4, 128, P, None, None) == NULL
    assert f(P + 2, 4, 128, P, P, None) == ALIGN
    assert f(P, 4, 128, P + 1, P, None) == ALIGN
    assert f(None, 0, 128, None, None, None) == OK  # M == 0: nothing to do


def test_gemm_rejects_bad_arguments():
    f = qoq.qoq_w4a8_gemm
    args = dict(x8=P, s_x=P, M=4, K=4096, packed=P, s1=P, N=4096, group=128, y=P,
                acc_debug=None, workspace=None, workspace_bytes=0, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(*a.values())

    assert call(group=64) == GROUP
    assert call(K=4000) == SHAPE
    assert call(N=4008) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(M=0) == OK
    for name in ("x8", "s_x", "packed", "s1", "y"):
        assert call(**{name: None}) == NULL, name
    assert call(x8=P + 1) == ALIGN
    assert call(packed=P + 8) == ALIGN
    M, N, K = 1, 4096, 4096
    need = qoq.qoq_gemm_workspace_bytes(M, N, K)
    if need:
        assert call(M=M, workspace=None, workspace_bytes=need) == WORKSPACE
        assert call(M=M, workspace=P, workspace_bytes=need - 1) == WORKSPACE
        assert call(M=M, workspace=P + 4, workspace_bytes=need) == ALIGN


def test_deep_narrow_layers_split_k_below_a_round_of_wide_tiles():
    # Qwen1.5-72B down (K = 24576, N = 8192): K in two ranges while its
    # 256 x 256 tiles are fewer than the CUs (M = 1024: 128 tiles, 1280: 160),
    # one range from a full round (M = 2048: 256 tiles)
    ws = [qoq.qoq_gemm_workspace_bytes(M, 8192, 24576) for M in (1024, 1280, 2048)]
    assert ws == [2 * 1024 * 8192 * 4, 2 * 1280 * 8192 * 4, 0]


def test_linear_workspace_bytes():
    # one fused launch (up to 12 tokens, K <= 8192, little repeated
    # quantization on this 4096-column layer): no workspace
    for M, K in [(1, 4096), (8, 8192), (8, 128), (9, 4096), (12, 8192)]:
        assert qoq.qoq_linear_workspace_bytes(M, 4096, K) == 0
    # otherwise x8 (tile layout) + token scales, each 256-byte aligned
    for M, K in [(9, 2048), (13, 4096), (16, 128), (64, 4096), (8, 14336), (4096, 4096)]:
        act = qoq.qoq_act_bytes(M, K)
        want = -(-act // 256) * 256 + -(-4 * M // 256) * 256
        assert qoq.qoq_linear_workspace_bytes(M, 4096, K) == want
    assert qoq.qoq_linear_workspace_bytes(0, 4096, 4096) == 0
    assert qoq.qoq_linear_workspace_bytes(4, 4000, 4096) == 0


def test_linear_path(monkeypatch):
    qoq.set_tuning("gemm", None)
    # one fused launch for M <= 8 with K <= 8192, otherwise two launches
    assert [qoq.qoq_linear_path(M, 4096, 4096) for M in (1, 8, 9, 12, 13, 64, 256)] == [1, 1, 1, 1, 0, 0, 0]
    # up to 12 tokens fused while M K ceil(N / 16) <= 64e6 (9-12 tokens only
    # for K >= 4096)
    assert [qoq.qoq_linear_path(1, N, 8192) for N in (24576, 49152)] == [1, 1]
    assert [qoq.qoq_linear_path(4, N, 8192) for N in (24576, 49152)] == [1, 0]
    assert [qoq.qoq_linear_path(8, N, 8192) for N in (8192, 15616, 15632, 24576, 49152)] == [1, 1, 0, 0, 0]
    assert [qoq.qoq_linear_path(8, N, 4096) for N in (14336, 28672)] == [1, 1]
    assert [qoq.qoq_linear_path(10, N, 4096) for N in (6144, 14336, 24992, 25008, 28672)] == [1, 1, 1, 0, 0]
    assert [qoq.qoq_linear_path(10, 8192, K) for K in (2048, 4096, 8192)] == [0, 1, 1]
    assert qoq.qoq_linear_path(8, 4096, 16384) == 0
    assert qoq.qoq_linear_path(0, 4096, 4096) == -1 and qoq.qoq_linear_path(4, 4008, 4096) == -1
    qoq.set_tuning("gemm", "fused,16")
    assert qoq.qoq_linear_path(16, 4096, 8192) == 1
    qoq.set_tuning("gemm", "decode,2,1,8,4")         # 2 row tiles, 13 column tiles
    assert qoq.qoq_linear_path(64, 208, 4096) == -1
    assert qoq.qoq_linear_path(64, 256, 4096) == 0


def test_linear_rejects_bad_arguments(monkeypatch):
    qoq.set_tuning("gemm", None)
    f = qoq.qoq_w4a8_linear
    args = dict(x=P, M=4, K=4096, packed=P, s1=P, N=4096, group=128, y=P,
                acc_debug=None, workspace=None, workspace_bytes=0, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(*a.values())

    assert call(group=64) == GROUP
    assert call(K=4000) == SHAPE
    assert call(N=4008) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(M=0) == OK
    for name in ("x", "packed", "s1", "y"):
        assert call(**{name: None}) == NULL, name
    assert call(x=P + 2) == ALIGN
    assert call(y=P + 2) == ALIGN
    need = qoq.qoq_linear_workspace_bytes(64, 4096, 4096)
    assert need > 0
    assert call(M=64) == WORKSPACE
    assert call(M=64, workspace=P, workspace_bytes=need - 1) == WORKSPACE
    assert call(M=64, workspace=P + 8, workspace_bytes=need) == ALIGN
    # the fused kernel cannot take 64 tokens: a forced fused configuration is refused
    qoq.set_tuning("gemm", "fused,8")
    assert call(M=64, workspace=P, workspace_bytes=need) == 8
    assert call(M=4, K=16384) == 8          # 128 groups do not fit 8 waves x 4 groups
    qoq.set_tuning("gemm", "fused,5")
    assert call() == 8


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        qoq.quantize_act(torch.zeros((2, 128), dtype=torch.float16))
    with pytest.raises(ValueError):
        qoq.pack_weights(torch.zeros((16, 128), dtype=torch.float32))


def test_unknown_kernel_override_is_rejected_before_launch(monkeypatch):
    f = qoq.qoq_w4a8_gemm
    for bad in ("tile32,99,1,1,1", "nonsense", "decode,9,9,9,9"):
        qoq.set_tuning("gemm", bad)
        assert f(P, P, 4, 4096, P, P, 4096, 128, P, None, None, 0, None) == 8
        assert qoq.qoq_gemm_workspace_bytes(4, 4096, 4096) == 0


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU: --gpus above 1 (or a multi-rank
    launch) exits with status 2 and a message, before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr and r.stdout == ""
    env["WORLD_SIZE"] = "4"
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py")],
                       capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr


def test_gemm_refuses_k_beyond_exact_accumulation():
    """K above 139648 could wrap the INT32 accumulators (K * 127 * 121 >= 2^31
    from there on): the GEMM entry points refuse it before any launch, the
    size queries return 0 / -1; W8A8 (weights within 127) stops at 133120."""
    K_ok, K_bad = 139648, 139648 + 128
    assert qoq.qoq_gemm_workspace_bytes(64, 4096, K_bad) == 0
    assert qoq.qoq_linear_workspace_bytes(64, 4096, K_bad) == 0
    assert qoq.qoq_linear_path(64, 4096, K_bad) == -1
    assert qoq.qoq_linear_path(64, 4096, K_ok) in (0, 1)
    assert qoq.qoq_w4a8_gemm(P, P, 8, K_bad, P, P, 4096, 128, P, None, None, 0, None) == SHAPE
    assert qoq.qoq_w4a8_gemm_noalloc(P, P, 8, K_bad, P, P, 4096, 128, P, None, None) == SHAPE
    assert qoq.qoq_w4a8_linear(P, 8, K_bad, P, P, 4096, 128, P, None, None, 0, None) == SHAPE
    assert qoq.lib().qoq_w8a8_gemm(P, P, 8, 133120 + 128, P, P, 4096, P, None, None) == SHAPE
    assert qoq.qoq_packed_weight_bytes(16, K_bad) > 0   # packing any K is fine


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="needs a host without a visible GPU: the launch must fail, not run")
def test_launch_failure_reports_hip_error():
    """With no GPU the host checks pass and the launch itself fails: every
    entry point returns QOQ_ERR_HIP (nothing runs; the pointers are never
    dereferenced)."""
    assert qoq.qoq_quantize_act(P, 4, 128, P, P, None) == HIP
    assert qoq.qoq_w4a8_gemm(P, P, 4, 128, P, P, 16, 128, P, None, None, 0, None) == HIP
    assert qoq.qoq_w4a8_linear(P, 4, 128, P, P, 16, 128, P, None, P, 1 << 20, None) == HIP
    assert qoq.qoq_pack_weights(P, 16, 128, 128, P, P, None, 0, None) == HIP
    # the allocation-free GEMM fails already when it looks up its scratch array
    assert qoq.qoq_w4a8_gemm_noalloc(P, P, 64, 16384, P, P, 4096, 128, P, None, None) == HIP


def test_tuning_keys_and_errors():
    """Plan overrides go through qoq_set_tuning only (no environment
    variable is read): unknown keys and a NULL key are refused; a set
    override is used by the next call and cleared by an empty value."""
    L = qoq.lib()
    assert L.qoq_set_tuning(None, b"x") == NULL
    assert L.qoq_set_tuning(b"nonsense", b"1") == 8
    os.environ["QOQ_GEMM_CONFIG"] = "nonsense"          # ignored by the library
    try:
        assert qoq.qoq_gemm_workspace_bytes(64, 528, 2560) == 0
        qoq.set_tuning("gemm", "lds,4,1,4,2,3")
        assert qoq.qoq_gemm_workspace_bytes(64, 528, 2560) == 3 * 64 * 528 * 4
        qoq.set_tuning("gemm", "")
        assert qoq.qoq_gemm_workspace_bytes(64, 528, 2560) == 0
    finally:
        del os.environ["QOQ_GEMM_CONFIG"]
        qoq.clear_tuning()
