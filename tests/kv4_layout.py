"""Decoder of the KV4 cache layout as include/qoq_kv4.h documents it (test
helper: reading the library's cache through it and comparing with the
oracle checks the layout as well as the codes)."""
import numpy as np

D = 128


def _pi(k):
    """token of k-index 8g + e in a 32-token block"""
    g, e = k // 8, k % 8
    return 4 * g + e if e < 4 else 16 + 4 * g + e - 4


def _word_codes(w):
    """uint32 words -> codes [..., 8]: element e at bit 4 (e // 2) + 16 (e % 2)."""
    w = w.astype(np.uint64)
    return np.stack([(w >> (4 * (e // 2) + 16 * (e % 2))) & 15 for e in range(8)],
                    axis=-1).astype(np.uint8)


def decode_cache(cache, B, Hkv, C):
    """dict(kc, ks, kz, vc, vs, vz) with codes [B, C, Hkv, D] uint8 and
    scale fp16 / zero uint16 [B, C, Hkv], from the raw cache bytes."""
    a = np.asarray(cache).reshape(B, Hkv, C * 133)
    nblk = C // 32
    out = {n: None for n in ("kc", "ks", "kz", "vc", "vs", "vz")}
    kc = np.zeros((B, C, Hkv, D), np.uint8)
    vc = np.zeros((B, C, Hkv, D), np.uint8)
    # key block [tile 2][g 4][t 16][word st 4] (uint32); element e of a word
    # at bit 4 (e // 2) + 16 (e % 2)
    kb = a[:, :, :nblk * 2048].copy().view(np.uint32).reshape(B, Hkv, nblk, 2, 4, 16, 4)
    codes = _word_codes(kb)                              # [..., st, e 0..7]
    # axes: B, Hkv, blk, tile, g, t, st, e -> token 32 blk + 16 tile + t, dim 32 st + 8 g + e
    codes = codes.transpose(0, 1, 2, 3, 5, 6, 4, 7).reshape(B, Hkv, C, D)
    kc[:] = codes.transpose(0, 2, 1, 3)
    # value block [g 4][d 16][c 8] (uint32): dim 16 c + d, k-index 8g + e
    vb = a[:, :, nblk * 2048:nblk * 4096].copy().view(np.uint32).reshape(B, Hkv, nblk, 4, 16, 8)
    vcodes = _word_codes(vb)                              # [B, Hkv, blk, g, d, c, e]
    tok = np.array([[_pi(8 * g + e) for e in range(8)] for g in range(4)])
    for g in range(4):
        for e in range(8):
            t = tok[g, e]
            # dims 16 c + d
            vals = vcodes[:, :, :, g, :, :, e]               # [B, Hkv, blk, d, c]
            vals = vals.transpose(0, 1, 2, 4, 3).reshape(B, Hkv, nblk, D)
            vc[:, t::32, :, :] = vals.transpose(0, 2, 1, 3)
    # metadata block (160 bytes): 32 fp16 s_k, 32 fp16 s_v, 32 bytes z_k | z_v << 4,
    # each in k order (token pi(k))
    mb = a[:, :, nblk * 4096:].reshape(B, Hkv, nblk, 160)
    order = np.array([_pi(k) for k in range(32)])
    sk = np.zeros((B, Hkv, nblk, 32), np.uint16)
    sv = np.zeros((B, Hkv, nblk, 32), np.uint16)
    zb = np.zeros((B, Hkv, nblk, 32), np.uint8)
    sk[..., order] = mb[..., :64].copy().view(np.uint16)
    sv[..., order] = mb[..., 64:128].copy().view(np.uint16)
    zb[..., order] = mb[..., 128:160]

    def tok(x):                                           # [B, Hkv, nblk, 32] -> [B, C, Hkv]
        return x.reshape(B, Hkv, C).transpose(0, 2, 1)
    out.update(kc=kc, vc=vc, ks=tok(sk).view(np.float16), vs=tok(sv).view(np.float16),
               kz=tok(zb & 15).astype(np.int64), vz=tok(zb >> 4).astype(np.int64))
    return out
