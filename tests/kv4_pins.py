"""Pins of the KV4 decode-attention oracle (oracle/kv4.py) to facts outside
it: hand-derived smoothing factors, codes, scales and zeros; closed forms of
softmax attention (one token, a zero query, two tokens with a chosen score
gap); the grouped-query head mapping; the length mask; the smoothing
identity (q lambda) . (k / lambda) = q . k; a pure-Python brute force.

Each pin takes the oracle module, so that planted mistakes in copies of it
(test_oracle_kv4_mutants.py) can be shown to fail at least one pin.

Hand-derived values (exact fp16 / fp32 arithmetic):
  * sqrt(4) = 2, sqrt(0.25) = 0.5, sqrt(9) = 3, sqrt(2) = 1.41421356... ->
    fp16 1.4140625 (1448 / 1024); an all-zero channel gets 1.
  * x = [3, -1.5, 0, ..., 0]: lo = -1.5, hi = 3, fp32(4.5 / 15) = 0.3 (fp32
    0.30000001192...) -> fp16 205/1024 * 1/4 = 0.300048828125; z = rne(1.5 /
    0.300048828125 = 4.99918...) = 5; codes rne(3 / s = 9.99837...) + 5 =
    15, rne(-4.99918...) + 5 = 0, 0 + 5 = 5; values (15 - 5) s =
    3.00048828125, (0 - 5) s = -1.500244140625, 0.
"""
import math

import numpy as np

D = 128
S_HAND = 0.300048828125


def _hand_vector():
    x = np.zeros(D, dtype=np.float32)
    x[0], x[1] = 3.0, -1.5
    return x


def pin_smooth_factors_hand(mod):
    k = np.zeros((3, 1, 5), dtype=np.float16)
    k[0, 0] = [4.0, 2.0, 0.0, 0.25, -9.0]
    k[1, 0] = [-1.0, 1.0, 0.0, -0.125, 2.0]
    k[2, 0] = [3.5, -2.0, 0.0, 0.25, 8.0]
    lam = mod.smooth_factors(k)
    assert lam.dtype == np.float16 and lam.shape == (1, 5)
    assert lam[0].tolist() == [2.0, 1.4140625, 1.0, 0.5, 3.0], lam


def pin_kv4_quantize_hand(mod):
    x = np.stack([_hand_vector(), np.zeros(D, np.float32)])
    codes, s, z = mod.kv4_quantize(x)
    assert s.dtype == np.float16 and float(s[0]) == S_HAND and float(s[1]) == 0.0
    assert int(z[0]) == 5 and int(z[1]) == 0
    assert int(codes[0, 0]) == 15 and int(codes[0, 1]) == 0 and np.all(codes[0, 2:] == 5)
    assert np.all(codes[1] == 0)
    deq = mod.kv4_dequantize(codes, s, z)
    assert deq[0, 0] == 10 * S_HAND and deq[0, 1] == -5 * S_HAND and np.all(deq[0, 2:] == 0)
    assert np.all(deq[1] == 0)


def pin_keys_divided_values_not(mod):
    """Keys are divided by lambda before quantization (2x the hand vector with
    lambda 2 gives the hand codes); values are quantized unsmoothed."""
    lam = np.full((1, D), 2.0, dtype=np.float16)
    k = (2 * _hand_vector()).astype(np.float16).reshape(1, 1, 1, D)
    v = _hand_vector().astype(np.float16).reshape(1, 1, 1, D)
    enc = mod.kv4_encode(k, v, lam)
    for p in ("k", "v"):
        assert float(enc[p + "s"].reshape(-1)[0]) == S_HAND, p
        assert int(enc[p + "z"].reshape(-1)[0]) == 5, p
        c = enc[p + "c"].reshape(-1)
        assert int(c[0]) == 15 and int(c[1]) == 0, p


def pin_query_multiplied_per_kv_head(mod):
    """q~ = fp16(q * lambda[h // group]): 4 query heads on 2 KV heads."""
    lam = np.ones((2, D), dtype=np.float16)
    lam[0, :] = 2.0
    lam[1, :] = 3.0
    lam[1, 5] = 0.5
    q = np.ones((1, 4, D), dtype=np.float16)
    q[0, 3, 5] = 0.1
    qs = mod.smooth_query(q, lam, 2)
    assert qs.dtype == np.float16
    assert np.all(qs[0, 0] == 2) and np.all(qs[0, 1] == 2)
    assert qs[0, 2, 0] == 3 and qs[0, 2, 5] == 0.5
    # fp32(fp16(0.1) * 0.5) rounded to fp16: halving is exact
    assert qs[0, 3, 5] == np.float16(0.1) * np.float16(0.5)


def _core(mod, q, k, v, lens, group=1):
    return mod.attention_core(q, k, v, lens, group)[0]


def pin_single_token_is_its_value(mod):
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, D))
    k = rng.standard_normal((1, 4, 1, D))
    v = rng.standard_normal((1, 4, 1, D))
    o = _core(mod, q, k, v, [1], group=2)
    assert np.array_equal(o[0, 0], v[0, 0, 0]) and np.array_equal(o[0, 1], v[0, 0, 0])


def pin_zero_query_is_mean(mod):
    rng = np.random.default_rng(2)
    k = rng.standard_normal((2, 7, 1, D))
    v = rng.standard_normal((2, 7, 1, D))
    q = np.zeros((2, 1, D))
    o = _core(mod, q, k, v, [7, 3])
    assert np.allclose(o[0, 0], v[0, :7, 0].mean(axis=0), rtol=0, atol=1e-12)
    assert np.allclose(o[1, 0], v[1, :3, 0].mean(axis=0), rtol=0, atol=1e-12)


def pin_two_tokens_closed_form(mod):
    """Scores 0 and ln 3 (q . k_1 = sqrt(D) ln 3): weights 1/4 and 3/4."""
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 2, 1, D))
    k[0, 1, 0, 0] = math.sqrt(D) * math.log(3.0)
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 2, 1, D))
    o = _core(mod, q, k, v, [2])
    assert np.allclose(o[0, 0], 0.25 * v[0, 0, 0] + 0.75 * v[0, 1, 0], rtol=0, atol=1e-12)


def pin_grouped_query_mapping(mod):
    """Query head h reads KV head h // group."""
    q = np.ones((1, 6, D))
    k = np.zeros((1, 1, 3, D))
    v = np.zeros((1, 1, 3, D))
    for h in range(3):
        v[0, 0, h, :] = h + 1
    o = _core(mod, q, k, v, [1], group=2)
    assert [float(o[0, h, 0]) for h in range(6)] == [1, 1, 2, 2, 3, 3]


def pin_length_mask(mod):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 6, 1, D))
    v = rng.standard_normal((1, 6, 1, D))
    o = _core(mod, q, k, v, [4])
    k2, v2 = k.copy(), v.copy()
    k2[0, 4:] = 50.0
    v2[0, 4:] = 1e6
    o2 = _core(mod, q, k2, v2, [4])
    assert np.array_equal(o, o2)
    o3 = _core(mod, q, k[:, :4], v[:, :4], [4])
    assert np.allclose(o, o3, rtol=0, atol=1e-15)
    assert np.all(_core(mod, q, k, v, [0]) == 0)


def pin_smoothing_identity(mod):
    """With exact arithmetic, scaling queries by lambda and keys by 1 / lambda
    leaves attention unchanged."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, D))
    k = rng.standard_normal((1, 5, 1, D))
    v = rng.standard_normal((1, 5, 1, D))
    lam = np.exp(rng.standard_normal(D))
    o = _core(mod, q, k, v, [5], group=2)
    os_ = _core(mod, q * lam, k / lam, v, [5], group=2)
    assert np.allclose(o, os_, rtol=0, atol=1e-12)


def pin_bound_terms(mod):
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 2, D))
    k = rng.standard_normal((2, 9, 1, D))
    v = rng.standard_normal((2, 9, 1, D))
    o, a, r = mod.attention_core(q, k, v, [9, 5], 2)
    for b in range(2):
        n = [9, 5][b]
        for h in range(2):
            assert np.all(np.abs(o[b, h]) <= a[b, h] + 1e-15)
            sc = np.abs(k[b, :n, 0] @ q[b, h]) / math.sqrt(D)
            assert sc.max() <= r[b, h] + 1e-12


def pin_brute_force_end_to_end(mod):
    """Tiny case through the whole oracle against plain Python loops on the
    stored codes (dequantization, smoothed query, scores, softmax)."""
    rng = np.random.default_rng(7)
    B, T, Hkv, group = 1, 3, 1, 2
    k = rng.standard_normal((B, T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((B, T, Hkv, D)).astype(np.float16)
    q = rng.standard_normal((B, Hkv * group, D)).astype(np.float16)
    lam = mod.smooth_factors(k)
    enc = mod.kv4_encode(k, v, lam)
    res = mod.kv4_decode_attention(q, lam, enc, [T], group)
    for h in range(Hkv * group):
        qs = [float(np.float16(np.float32(q[0, h, d]) * np.float32(lam[h // group, d])))
              for d in range(D)]
        sc = []
        for t in range(T):
            s, z = float(enc["ks"][0, t, 0]), int(enc["kz"][0, t, 0])
            sc.append(sum(qs[d] * (int(enc["kc"][0, t, 0, d]) - z) * s for d in range(D)) / math.sqrt(D))
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        for d in (0, 17, 127):
            acc = 0.0
            for t in range(T):
                s, z = float(enc["vs"][0, t, 0]), int(enc["vz"][0, t, 0])
                acc += w[t] * (int(enc["vc"][0, t, 0, d]) - z) * s
            assert abs(acc / sum(w) - res["o"][0, h, d]) <= 1e-12, (h, d)


def pin_fp16_path_is_plain_attention(mod):
    """The fp16 comparison path: one token gives its value; a zero query the
    mean of the first len values."""
    rng = np.random.default_rng(8)
    k = rng.standard_normal((2, 5, 1, D)).astype(np.float16)
    v = rng.standard_normal((2, 5, 1, D)).astype(np.float16)
    q = rng.standard_normal((2, 2, D)).astype(np.float16)
    res = mod.fp16_decode_attention(q, k, v, [1, 5], 2)
    assert np.array_equal(res["o"][0, 0], v[0, 0, 0].astype(np.float64))
    q0 = np.zeros_like(q)
    res = mod.fp16_decode_attention(q0, k, v, [1, 5], 2)
    assert np.allclose(res["o"][1, 1], v[1, :, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)


KV4_PINS = [pin_smooth_factors_hand, pin_kv4_quantize_hand, pin_keys_divided_values_not,
            pin_query_multiplied_per_kv_head, pin_single_token_is_its_value,
            pin_zero_query_is_mean, pin_two_tokens_closed_form, pin_grouped_query_mapping,
            pin_length_mask, pin_smoothing_identity, pin_bound_terms, pin_brute_force_end_to_end,
            pin_fp16_path_is_plain_attention]
