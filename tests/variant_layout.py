"""Decoders of the comparison GEMMs' buffer layouts as include/qoq_variants.h
documents them (test helpers: reading the library's buffers through these
and comparing with the oracle checks the layouts as well as the codes)."""
import numpy as np


def w8_codes(packed, N, K):
    """int8 codes [N, K] from the W8A8 packed weights
    [N/16][K/128][2 halves][64 lanes (c + 16h)][16 bytes]."""
    a = np.asarray(packed).view(np.int8).reshape(N // 16, K // 128, 2, 4, 16, 16)
    # axes: nb, g, s, h, c, b -> channel 16nb + c, input 128g + 64s + 16h + b
    return a.transpose(0, 4, 1, 2, 3, 5).reshape(N, K)


def w4_codes_scales(packed, N, K):
    """(codes int8 [N, K], scale fp16 [N, K/128]) from the W4A4 packed weights:
    the W4A8 nibble layout with u = code + 8, fp16 scales in the record slots."""
    p = np.asarray(packed)
    ng = K // 128
    nib = p[:N * K // 2].reshape(N // 16, ng, 4, 16, 16)     # nb, g, h, c, b
    lo = (nib & 15).astype(np.int16) - 8                      # input 16h + b
    hi = (nib >> 4).astype(np.int16) - 8                      # input 64 + 16h + b
    codes = np.concatenate([lo.transpose(0, 3, 1, 2, 4), hi.transpose(0, 3, 1, 2, 4)], axis=3)
    codes = codes.reshape(N // 16, 16, ng, 128).reshape(N, K).astype(np.int8)
    ng8 = -(-ng // 8)
    rec = p[N * K // 2:].view(np.uint16).reshape(N // 16, ng8, 16, 8)   # nb, chunk, c, g%8
    sc = rec.transpose(0, 2, 1, 3).reshape(N, ng8 * 8)[:, :ng].view(np.float16)
    return codes, sc


def x4_codes_scales(act, M, K):
    """(codes int8 [M, K], s_a float32 [M, K/128]) from a W4A4 activation
    buffer: x4 tile layout, then fp32 scales [K/128][M padded to 128]."""
    a = np.asarray(act)
    Mt = -(-M // 16) * 16
    x4 = a[:Mt * K // 2].reshape(Mt // 16, K // 16, 16, 8)   # tile, chunk j, row, byte b
    lo = (x4 & 15).astype(np.int16) - 8                      # input 16j + b
    hi = (x4 >> 4).astype(np.int16) - 8                      # input 16j + 8 + b
    codes = np.concatenate([lo, hi], axis=3)                 # tile, j, row, 16
    codes = codes.transpose(0, 2, 1, 3).reshape(Mt, K)[:M].astype(np.int8)
    off = -(-(Mt * K // 2) // 256) * 256
    Mp = -(-M // 128) * 128
    s_a = a[off:off + (K // 128) * Mp * 4].view(np.float32).reshape(K // 128, Mp)[:, :M].T
    return codes, s_a


def w4a16_codes_scales_zeros(packed, N, K):
    """(q uint8 [N, K], s fp16 [N, K/128], z uint16 [N, K/128]) from the W4A16
    packed weights: the W4A8 nibble layout with u = q, then the fp16 scales
    and the zeros (uint16) in two regions of the record shape."""
    p = np.asarray(packed)
    ng = K // 128
    nib = p[:N * K // 2].reshape(N // 16, ng, 4, 16, 16)     # nb, g, h, c, b
    lo = nib & 15                                             # input 16h + b
    hi = nib >> 4                                             # input 64 + 16h + b
    q = np.concatenate([lo.transpose(0, 3, 1, 2, 4), hi.transpose(0, 3, 1, 2, 4)], axis=3)
    q = q.reshape(N, K).astype(np.uint8)
    ng8 = -(-ng // 8)
    rb = N * ng8 * 16
    recs = []
    for r in range(2):
        rec = p[N * K // 2 + r * rb:N * K // 2 + (r + 1) * rb].view(np.uint16)
        rec = rec.reshape(N // 16, ng8, 16, 8).transpose(0, 2, 1, 3).reshape(N, ng8 * 8)
        recs.append(rec[:, :ng])
    return q, recs[0].view(np.float16), recs[1]
