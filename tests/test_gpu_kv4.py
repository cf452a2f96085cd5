"""KV4 decode attention with SmoothAttention scaling against its oracle.

Smoothing factors, cache codes, scales and zeros bit-exact (read through
the documented layout, after appends that start mid-block and append one
token at a time); the attention output within the error bound of its fp32
scores, fp16 probabilities and fp16 dequantized values; exact cases
(one-token contexts give the dequantized value bit for bit, empty contexts
give 0); every split of the contexts; the three benchmarked workloads at
full size on every head.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from kv4_layout import decode_cache

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.uint16)).view(torch.float16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def _factors(k_calib):
    """Smoothing factors from the same calibration keys on both sides: the
    library's (device) and the oracle's (host), which must agree bit for bit."""
    lam_d = qoq.kv4_smooth_factors(_dev(k_calib))
    lam = oracle.smooth_factors(k_calib)
    torch.cuda.synchronize()
    assert np.array_equal(lam_d.cpu().numpy().view(np.uint16), lam.view(np.uint16))
    return lam, lam_d


def _build(B, H, Hkv, lens, C, seed, chunks=None):
    """Cache filled through qoq_kv4_append (optionally in several calls);
    returns (q, k, v, lam (oracle), lam_d (library), cache_d)."""
    q, k, v = wl.make_attention(B, H, Hkv, D, lens, seed=seed)
    T = k.shape[1]
    lam, lam_d = _factors(k.reshape(-1, Hkv, D))
    cache = qoq.kv4_alloc_cache(B, Hkv, C, DEV)
    cache.fill_(0xAB)                      # never-written tokens hold garbage
    bounds = chunks or [T]
    pos = 0
    for end in bounds:
        n = end - pos
        if n > 0:
            start = _dev(np.full(B, pos, np.int32))
            qoq.kv4_append(_dev(k[:, pos:end]), _dev(v[:, pos:end]), lam_d, start, cache, C)
        pos = end
    torch.cuda.synchronize()
    return q, k, v, lam, lam_d, cache


def _check_cache(cache, k, v, lam, B, Hkv, C, T):
    got = decode_cache(cache.cpu().numpy(), B, Hkv, C)
    ref = oracle.kv4_encode(k, v, lam)
    for n in ("kc", "vc"):
        assert np.array_equal(got[n][:, :T], ref[n]), n
    for n in ("ks", "vs"):
        assert np.array_equal(got[n][:, :T].view(np.uint16), ref[n].view(np.uint16)), n
    for n in ("kz", "vz"):
        assert np.array_equal(got[n][:, :T].astype(np.int64), ref[n].astype(np.int64)), n
    return ref


def _tolerance(ref, res, lens):
    """|o - o_exact| bound per output: fp16 output rounding, fp16 values and
    probabilities, fp32 accumulation over the context, and score errors
    (fp32 sums of 128 products and of the query) moving the weights."""
    qs = res["qs"].astype(np.float64)                     # [B, H, D]
    B, H, _ = qs.shape
    Hkv = ref["ks"].shape[2]
    G = H // Hkv
    tol = np.zeros((B, H, D))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(H):
            sk = np.abs(ref["ks"][b, :n, h // G].astype(np.float64)).max()
            dz = sk * np.abs(qs[b, h]).sum() * 2.0 ** -12 / math.sqrt(D)
            rel = 2.0 ** -10 + (n + 64) * 2.0 ** -23 + 2.0 * dz
            tol[b, h] = 2.0 ** -11 * np.abs(res["o"][b, h]) + rel * res["a"][b, h] + 2.0 ** -24
    return tol


def _run(B, H, Hkv, lens, C, seed, monkeypatch, splits=None, chunks=None):
    qoq.set_tuning("kv4_splits", None)
    if splits:
        qoq.set_tuning("kv4_splits", str(splits))
    print(f"\n[gpu-case] kv4 B={B} H={H} Hkv={Hkv} lens={list(lens)} C={C} splits={splits} "
          f"paired={qoq.get_tuning('kv4_paired') or 'default'}",
          flush=True)
    q, k, v, lam, lam_d, cache = _build(B, H, Hkv, lens, C, seed, chunks)
    T = k.shape[1]
    ref = _check_cache(cache, k, v, lam, B, Hkv, C, T)
    res = oracle.kv4_decode_attention(q, lam, ref, lens, H // Hkv)
    o = qoq.kv4_decode_attention(_dev(q), lam_d, cache, C, _dev(np.asarray(lens, np.int32)),
                                 int(max(lens)), Hkv)
    torch.cuda.synchronize()
    got = o.cpu().float().numpy().astype(np.float64)
    tol = _tolerance(ref, res, lens)
    bad = np.abs(got - res["o"]) > tol
    assert not bad.any(), (f"{bad.sum()} outputs outside the bound, first at {np.argwhere(bad)[:3]}, "
                           f"err {np.abs(got - res['o'])[bad][:3]}, tol {tol[bad][:3]}")
    return got, res, ref


@pytest.mark.parametrize("fp16", [False, True])
def test_cache_offsets_beyond_2_32(fp16, monkeypatch):
    """A cache of 2^21 tokens per (sequence, KV head): the last regions start
    more than 4 GiB into the buffer (64-bit region offsets); short contexts
    keep the oracle small. Appended at the start of every region and, for the
    second sequence, at the far end of its capacity."""
    qoq.set_tuning("kv4_splits", None)
    B, H, Hkv, C = 2, 32, 8, 1 << 21
    lens = np.array([50, 77], np.int32)
    print(f"\n[gpu-case] kv{'16' if fp16 else '4'} capacity 2^21 B={B} Hkv={Hkv}", flush=True)
    q, k, v = wl.make_attention(B, H, Hkv, D, lens, seed=23)
    lam, lam_d = _factors(k.reshape(-1, Hkv, D))
    if fp16:
        cache = qoq.kv16_alloc_cache(B, Hkv, C, DEV)
        assert cache.numel() > (1 << 33)
        qoq.kv16_append(_dev(k), _dev(v), _dev(np.zeros(B, np.int32)), cache, C)
        # the same tokens again at the far end of the capacity (never read)
        qoq.kv16_append(_dev(k), _dev(v), _dev(np.full(B, C - k.shape[1], np.int32)), cache, C)
        o = qoq.kv16_decode_attention(_dev(q), cache, C, _dev(lens), int(lens.max()), Hkv)
        res = oracle.fp16_decode_attention(q, k, v, lens, H // Hkv)
        torch.cuda.synchronize()
        got = o.cpu().float().numpy().astype(np.float64)
        for b, n in enumerate(lens):
            rel = 2.0 ** -10 + (n + 64) * 2.0 ** -23 + 2.0 * (D + 8) * 2.0 ** -24 * res["r"][b][:, None]
            tol = 2.0 ** -11 * np.abs(res["o"][b]) + rel * res["a"][b] + 2.0 ** -24
            assert np.all(np.abs(got[b] - res["o"][b]) <= tol), b
        return
    cache = qoq.kv4_alloc_cache(B, Hkv, C, DEV)
    assert cache.numel() > (1 << 32)
    qoq.kv4_append(_dev(k), _dev(v), lam_d, _dev(np.zeros(B, np.int32)), cache, C)
    qoq.kv4_append(_dev(k), _dev(v), lam_d, _dev(np.full(B, C - k.shape[1], np.int32)), cache, C)
    o = qoq.kv4_decode_attention(_dev(q), lam_d, cache, C, _dev(lens), int(lens.max()), Hkv)
    torch.cuda.synchronize()
    enc = oracle.kv4_encode(k, v, lam)
    res = oracle.kv4_decode_attention(q, lam, enc, lens, H // Hkv)
    got = o.cpu().float().numpy().astype(np.float64)
    tol = _tolerance(enc, res, lens)
    assert np.all(np.abs(got - res["o"]) <= tol)


def test_smooth_factors_exact():
    rng = np.random.default_rng(3)
    kc = (rng.standard_normal((300, 4, D)) * np.exp(rng.standard_normal((1, 4, D)))).astype(np.float16)
    kc[:, 1, 7] = 0
    kc[:, 2, 9] = np.float16(-3.0)
    lam = qoq.kv4_smooth_factors(_dev(kc))
    torch.cuda.synchronize()
    ref = oracle.smooth_factors(kc)
    assert np.array_equal(lam.cpu().numpy().view(np.uint16), ref.view(np.uint16))
    assert float(ref[1, 7]) == 1.0


@pytest.mark.parametrize("B,H,Hkv,lens,C", [
    (3, 8, 2, [1, 33, 100], 128),          # ragged, partial blocks
    (2, 4, 4, [64, 31], 64),               # no grouping (G = 1)
    (2, 16, 1, [200, 5], 256),             # 16 query heads on one KV head
    (4, 32, 8, [90, 0, 17, 128], 128),     # an empty context
])
def test_attention_parity(B, H, Hkv, lens, C, monkeypatch):
    got, res, _ = _run(B, H, Hkv, lens, C, seed=B + H + C, monkeypatch=monkeypatch)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("paired", ["1", "0"])
@pytest.mark.parametrize("B,H,Hkv,lens,C", [
    (5, 8, 2, [40, 128, 3, 128, 77], 128),     # odd batch (the middle rank runs alone), a tie
    (6, 4, 1, [0, 96, 1, 64, 95, 96], 96),      # empty context, ties, one-token context
    (2, 32, 8, [128, 17], 128),                 # one pair
    (4, 8, 2, [0, 0, 0, 1200], 1216),           # a pair of two empty contexts
])
def test_paired_schedule(B, H, Hkv, lens, C, paired, monkeypatch):
    """Unsplit batches of 2..256 sequences whose pairs fit one per CU run two
    contexts of complementary length rank per 8-wave workgroup; the same
    cases with the schedule turned off meet the same bound."""
    qoq.set_tuning("kv4_paired", paired)
    got, res, _ = _run(B, H, Hkv, lens, C, seed=B + 3 * H + C, monkeypatch=monkeypatch)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("paired", ["1", "0"])
def test_blocks_per_wave(paired, monkeypatch):
    """Whole contexts per workgroup (one split), in the paired schedule's
    8-wave workgroups and in 4-wave ones, on contexts of 0 to 48 blocks:
    waves run none to several whole rounds of the block ring and end with
    any number of blocks left in it, and the last block of a context is
    full or partial."""
    qoq.set_tuning("kv4_paired", paired)
    _run(8, 8, 2, [0, 1, 100, 257, 500, 800, 1100, 1530], 1536, seed=41,
         monkeypatch=monkeypatch, splits=1)


def test_many_splits_merge(monkeypatch):
    """More than 16 splits of one context (one block each): the merge reads
    its splits in rounds of eight instead of all at once."""
    _run(2, 8, 2, [600, 100], 640, seed=19, monkeypatch=monkeypatch, splits=32)


@pytest.mark.parametrize("B,H,Hkv,lens,C,splits", [
    # one long context among empty and short ones: most splits of the short
    # contexts hold no block, an empty context's merge reads none
    (5, 8, 2, [2000, 0, 33, 1, 700], 2016, 4),
    (3, 16, 4, [1500, 20, 900], 1504, 12),
    # every context empty or one token
    (4, 8, 1, [0, 1, 0, 1], 32, 3),
    # more contexts than a wave has lanes
    (100, 4, 1, [int(x) for x in np.random.default_rng(5).integers(0, 200, 100)], 224, 3),
])
def test_splits_of_ragged_contexts(B, H, Hkv, lens, C, splits, monkeypatch):
    """Contexts of very different lengths cut into the same number of
    splits, sized by the longest: splits past a context's end write nothing
    and the merge reads only those that hold tokens."""
    _run(B, H, Hkv, lens, C, seed=37, monkeypatch=monkeypatch, splits=splits)


@pytest.mark.parametrize("B,H,Hkv,lens,C,splits", [
    (4, 4, 4, [300, 0, 1, 257], 320, 3),                       # G = 1
    (2, 64, 4, [500, 33], 512, 5),                             # G = 16
    (2, 8, 4, [1200, 0], 1216, 20),                            # more than 16 splits
    (8, 8, 1, [0, 1, 31, 32, 33, 500, 1, 0], 512, 4),          # G = 8, empty and one-token
])
def test_splits_merged_on_the_regions_xcd(B, H, Hkv, lens, C, splits, monkeypatch):
    """Split batches whose (sequence, KV head) regions come in whole rounds
    of 8: the splits of a region and the one-wave merge workgroups of its
    rows are numbered onto the same XCD."""
    assert (B * Hkv) % 8 == 0
    _run(B, H, Hkv, lens, C, seed=43, monkeypatch=monkeypatch, splits=splits)


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_attention_every_split(splits, monkeypatch):
    _run(3, 8, 2, [300, 45, 257], 320, seed=17, monkeypatch=monkeypatch, splits=splits)


def test_appends_in_pieces(monkeypatch):
    """Appends that start mid-block, then single tokens (decode steps): the
    cache equals one append of everything."""
    _run(2, 8, 2, [70, 70], 96, seed=23, monkeypatch=monkeypatch, chunks=[13, 45, 46, 47, 70])


def test_single_token_context_is_exact(monkeypatch):
    """One cached token: the output is its dequantized value fp16((u - z) s)
    bit for bit, whatever the query."""
    qoq.set_tuning("kv4_splits", None)
    B, H, Hkv, C = 3, 8, 2, 32
    q, k, v, lam, lam_d, cache = _build(B, H, Hkv, [1, 1, 1], C, seed=29)
    ref = oracle.kv4_encode(k, v, lam)
    o = qoq.kv4_decode_attention(_dev(q), lam_d, cache, C, _dev(np.ones(B, np.int32)), 1, Hkv)
    torch.cuda.synchronize()
    vh = oracle.kv4_dequantize(ref["vc"], ref["vs"], ref["vz"]).astype(np.float16)   # [B, 1, Hkv, D]
    want = np.repeat(vh[:, 0], H // Hkv, axis=1)
    assert np.array_equal(o.cpu().numpy().view(np.uint16), want.view(np.uint16))


def test_zero_query_is_mean(monkeypatch):
    qoq.set_tuning("kv4_splits", None)
    B, H, Hkv, C = 2, 4, 2, 128
    lens = [100, 37]
    q, k, v, lam, lam_d, cache = _build(B, H, Hkv, lens, C, seed=31)
    q[:] = 0
    ref = oracle.kv4_encode(k, v, lam)
    o = qoq.kv4_decode_attention(_dev(q), lam_d, cache, C, _dev(np.asarray(lens, np.int32)), 100, Hkv)
    torch.cuda.synchronize()
    vh = oracle.kv4_dequantize(ref["vc"], ref["vs"], ref["vz"])
    got = o.cpu().float().numpy().astype(np.float64)
    for b, n in enumerate(lens):
        for h in range(H):
            mean = vh[b, :n, h // 2].mean(axis=0)
            a = np.abs(vh[b, :n, h // 2]).mean(axis=0)
            assert np.all(np.abs(got[b, h] - mean) <= 2.0 ** -11 * np.abs(mean) + 2.0 ** -9 * a + 1e-7)


@pytest.mark.parametrize("key", list(wl.ATTN_WORKLOADS))
def test_workload_every_head(key, monkeypatch):
    """Every attention workload the benchmark times (Llama-3-8B-shaped: 64
    sequences of 512-2048 tokens; Qwen1.5-72B-shaped: 16 x 64 heads; long
    contexts of 8-16 K tokens, split over workgroups) at full size, in the
    benchmark's launch configuration, for the 4-bit and the fp16 cache; the
    oracle checks every sequence and head, one sequence at a time."""
    qoq.set_tuning("kv4_splits", None)
    w = wl.ATTN_WORKLOADS[key]
    q, k, v, lens = wl.make_attention_case(w)
    C = int(-(-lens.max() // 32) * 32)
    max_len = int(lens.max())
    print(f"\n[gpu-case] kv4 workload {key} B={w.B} H={w.H} Hkv={w.H_kv} C={C}", flush=True)
    lam, lam_d = _factors(k[:4].reshape(-1, w.H_kv, D))
    zeros = _dev(np.zeros(w.B, np.int32))
    kd, vd = _dev(k), _dev(v)
    cache = qoq.kv4_alloc_cache(w.B, w.H_kv, C, DEV)
    qoq.kv4_append(kd, vd, lam_d, zeros, cache, C)
    o = qoq.kv4_decode_attention(_dev(q), lam_d, cache, C, _dev(lens), max_len, w.H_kv)
    del cache
    cache16 = qoq.kv16_alloc_cache(w.B, w.H_kv, C, DEV)
    qoq.kv16_append(kd, vd, zeros, cache16, C)
    o16 = qoq.kv16_decode_attention(_dev(q), cache16, C, _dev(lens), max_len, w.H_kv)
    torch.cuda.synchronize()
    del cache16, kd, vd
    got = o.cpu().float().numpy().astype(np.float64)
    got16 = o16.cpu().float().numpy().astype(np.float64)
    G = w.H // w.H_kv
    for b in range(w.B):
        n = int(lens[b])
        sub = dict(k=k[b:b + 1, :n], v=v[b:b + 1, :n])
        enc = oracle.kv4_encode(sub["k"], sub["v"], lam)
        res = oracle.kv4_decode_attention(q[b:b + 1], lam, enc, [n], G)
        tol = _tolerance(enc, res, [n])
        assert np.all(np.abs(got[b:b + 1] - res["o"]) <= tol), ("kv4", b)
        res16 = oracle.fp16_decode_attention(q[b:b + 1], sub["k"], sub["v"], [n], G)
        rel = 2.0 ** -10 + (n + 64) * 2.0 ** -23 + 2.0 * (D + 8) * 2.0 ** -24 * res16["r"][0][:, None]
        tol16 = 2.0 ** -11 * np.abs(res16["o"][0]) + rel * res16["a"][0] + 2.0 ** -24
        assert np.all(np.abs(got16[b] - res16["o"][0]) <= tol16), ("fp16", b)


# ---------------------------------------------------------------------------
# the fp16 comparison path
# ---------------------------------------------------------------------------
def _run16(B, H, Hkv, lens, C, seed, monkeypatch, splits=None):
    qoq.set_tuning("kv4_splits", None)
    if splits:
        qoq.set_tuning("kv4_splits", str(splits))
    print(f"\n[gpu-case] kv16 B={B} H={H} Hkv={Hkv} lens={list(lens)} C={C} splits={splits} "
          f"paired={qoq.get_tuning('kv4_paired') or 'default'}",
          flush=True)
    q, k, v = wl.make_attention(B, H, Hkv, D, lens, seed=seed)
    cache = qoq.kv16_alloc_cache(B, Hkv, C, DEV)
    cache.fill_(0xFF)                      # never-written tokens hold NaN bit patterns
    qoq.kv16_append(_dev(k), _dev(v), _dev(np.zeros(B, np.int32)), cache, C)
    o = qoq.kv16_decode_attention(_dev(q), cache, C, _dev(np.asarray(lens, np.int32)),
                                  int(max(lens)), Hkv)
    torch.cuda.synchronize()
    res = oracle.fp16_decode_attention(q, k, v, lens, H // Hkv)
    got = o.cpu().float().numpy().astype(np.float64)
    tol = np.zeros_like(got)
    for b, n in enumerate(lens):
        for h in range(H):
            rel = 2.0 ** -10 + (n + 64) * 2.0 ** -23 + 2.0 * (D + 8) * 2.0 ** -24 * res["r"][b, h]
            tol[b, h] = 2.0 ** -11 * np.abs(res["o"][b, h]) + rel * res["a"][b, h] + 2.0 ** -24
    bad = np.abs(got - res["o"]) > tol
    assert not bad.any(), f"{bad.sum()} outputs outside the bound, first at {np.argwhere(bad)[:3]}"
    return got, v


@pytest.mark.parametrize("B,H,Hkv,lens,C", [(3, 8, 2, [1, 33, 100], 128), (2, 4, 4, [64, 31], 64),
                                            (4, 32, 8, [90, 0, 17, 128], 128)])
def test_fp16_attention_parity(B, H, Hkv, lens, C, monkeypatch):
    got, _ = _run16(B, H, Hkv, lens, C, seed=41 + B, monkeypatch=monkeypatch)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("paired", ["1", "0"])
def test_fp16_paired_schedule(paired, monkeypatch):
    qoq.set_tuning("kv4_paired", paired)
    _run16(5, 8, 2, [40, 128, 3, 128, 77], 128, seed=31, monkeypatch=monkeypatch)


@pytest.mark.parametrize("splits", [2, 5])
def test_fp16_attention_splits(splits, monkeypatch):
    _run16(3, 8, 2, [300, 45, 257], 320, seed=43, monkeypatch=monkeypatch, splits=splits)


def test_fp16_splits_of_ragged_contexts(monkeypatch):
    _run16(5, 8, 2, [2000, 0, 33, 1, 700], 2016, seed=47, monkeypatch=monkeypatch, splits=4)


def test_fp16_single_token_is_exact(monkeypatch):
    got, v = _run16(2, 8, 2, [1, 1], 32, seed=47, monkeypatch=monkeypatch)
    want = np.repeat(v[:, 0].astype(np.float64), 4, axis=1)
    assert np.array_equal(got, want)
