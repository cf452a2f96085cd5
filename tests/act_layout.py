"""The activation tile layout as the C header documents it, restated for the
tests: code (m, k) of an M x K activation matrix sits at byte
((m // 16) * (K // 16) + k // 16) * 256 + (m % 16) * 16 + k % 16.
Comparing the library's x8 buffer, read through these functions, with the
oracle's row-major codes checks the layout as well as the codes."""
import numpy as np


def act_rows(x8, M):
    """Row-major [M, K] codes (numpy int8) from an x8 buffer of shape
    (ceil(M/16), K/16, 16, 16) in the tile layout (torch or numpy)."""
    a = x8.cpu().numpy() if hasattr(x8, "cpu") else np.asarray(x8)
    T, J = a.shape[0], a.shape[1]
    return a.transpose(0, 2, 1, 3).reshape(T * 16, J * 16)[:M]


def act_offset(m, k, K):
    return ((m // 16) * (K // 16) + k // 16) * 256 + (m % 16) * 16 + k % 16
