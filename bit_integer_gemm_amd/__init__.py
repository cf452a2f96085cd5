"""Python binding of libqoq (QoQ W4A8 GEMM for MI355X / gfx950).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every computation runs in the HIP kernels of
``libqoq.so``. There is no CPU fallback: if the library is missing or no GPU
is visible the calls raise.

Low-level names mirror the C ABI in include/qoq.h (``qoq_pack_weights``,
``qoq_quantize_act``, ``qoq_w4a8_gemm``, ``qoq_packed_weight_bytes``,
``qoq_act_bytes``, ``qoq_gemm_workspace_bytes``, ``qoq_w4a8_linear``,
``qoq_linear_workspace_bytes``, ``qoq_status_string``); ``pack_weights``,
``quantize_act``, ``w4a8_gemm`` and ``w4a8_linear`` are the tensor-level
conveniences.

The INT8 activations travel in the library's activation tile layout: a
tensor of shape (ceil(M/16), K/16, 16, 16) whose element [t, j, r, b] is the
code of token 16t + r, input 16j + b (rows past M are never written).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "QoQError", "lib", "GROUP", "PACK_FROM_CANONICAL",
    "qoq_packed_weight_bytes", "qoq_act_bytes", "qoq_gemm_workspace_bytes", "qoq_pack_weights",
    "qoq_quantize_act", "qoq_w4a8_gemm", "qoq_w4a8_gemm_noalloc", "NOALLOC_SCRATCH_BYTES",
    "qoq_status_string", "qoq_w4a8_linear",
    "qoq_linear_workspace_bytes", "qoq_linear_path",
    "PackedWeight", "pack_weights", "pack_canonical", "quantize_act", "w4a8_gemm",
    "Workspace", "empty_act", "w4a8_linear",
    "w8a8_pack_weights", "w8a8_gemm", "w4a4_pack_weights", "w4a4_quantize_act", "w4a4_gemm",
    "w4a16_pack_weights", "w4a16_gemm",
    "kv4_cache_bytes", "kv4_alloc_cache", "kv4_smooth_factors", "kv4_append",
    "kv4_decode_attention", "kv16_alloc_cache", "kv16_append", "kv16_decode_attention",
    "qoq_stream_read", "set_tuning", "get_tuning", "clear_tuning", "TUNING_KEYS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqoq.so")
GROUP = 128
PACK_FROM_CANONICAL = 0x1

QOQ_STATUS = {
    0: "QOQ_OK", 1: "QOQ_ERR_NULL", 2: "QOQ_ERR_SHAPE", 3: "QOQ_ERR_ALIGN",
    4: "QOQ_ERR_GROUP", 5: "QOQ_ERR_WORKSPACE", 6: "QOQ_ERR_HIP", 7: "QOQ_ERR_FLAGS",
    8: "QOQ_ERR_CONFIG",
}


class QoQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {QOQ_STATUS.get(status, status)} "
                         f"({qoq_status_string(status)})")


class _Canonical(ctypes.Structure):
    _fields_ = [("q4", ctypes.c_void_p), ("s2", ctypes.c_void_p), ("z", ctypes.c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libqoq.so (built in-tree by ``python -m bit_integer_gemm_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_integer_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_uint32, ctypes.c_size_t)
        L.qoq_packed_weight_bytes.argtypes = [i64, i64, i32]
        L.qoq_packed_weight_bytes.restype = sz
        L.qoq_act_bytes.argtypes = [i64, i64]
        L.qoq_act_bytes.restype = sz
        L.qoq_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.qoq_gemm_workspace_bytes.restype = sz
        L.qoq_pack_weights.argtypes = [vp, i64, i64, i32, vp, vp, ctypes.POINTER(_Canonical),
                                       u32, vp]
        L.qoq_pack_weights.restype = ctypes.c_int
        L.qoq_quantize_act.argtypes = [vp, i64, i64, vp, vp, vp]
        L.qoq_quantize_act.restype = ctypes.c_int
        L.qoq_w4a8_gemm.argtypes = [vp, vp, i64, i64, vp, vp, i64, i32, vp, vp, vp, sz, vp]
        L.qoq_w4a8_gemm.restype = ctypes.c_int
        L.qoq_w4a8_gemm_noalloc.argtypes = [vp, vp, i64, i64, vp, vp, i64, i32, vp, vp, vp]
        L.qoq_w4a8_gemm_noalloc.restype = ctypes.c_int
        L.qoq_linear_workspace_bytes.argtypes = [i64, i64, i64]
        L.qoq_linear_workspace_bytes.restype = sz
        L.qoq_w4a8_linear.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp, vp, vp, sz, vp]
        L.qoq_w4a8_linear.restype = ctypes.c_int
        L.qoq_linear_path.argtypes = [i64, i64, i64]
        L.qoq_linear_path.restype = ctypes.c_int
        # comparison GEMMs (include/qoq_variants.h)
        L.qoq_w8a8_weight_bytes.argtypes = [i64, i64]
        L.qoq_w8a8_weight_bytes.restype = sz
        L.qoq_w8a8_pack_weights.argtypes = [vp, i64, i64, vp, vp, vp]
        L.qoq_w8a8_pack_weights.restype = ctypes.c_int
        L.qoq_w8a8_gemm.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp]
        L.qoq_w8a8_gemm.restype = ctypes.c_int
        L.qoq_w4a4_weight_bytes.argtypes = [i64, i64]
        L.qoq_w4a4_weight_bytes.restype = sz
        L.qoq_w4a4_act_bytes.argtypes = [i64, i64]
        L.qoq_w4a4_act_bytes.restype = sz
        L.qoq_w4a4_pack_weights.argtypes = [vp, i64, i64, vp, vp]
        L.qoq_w4a4_pack_weights.restype = ctypes.c_int
        L.qoq_w4a4_quantize_act.argtypes = [vp, i64, i64, vp, vp]
        L.qoq_w4a4_quantize_act.restype = ctypes.c_int
        L.qoq_w4a4_gemm.argtypes = [vp, i64, i64, vp, i64, vp, vp]
        L.qoq_w4a4_gemm.restype = ctypes.c_int
        # KV4 decode attention (include/qoq_kv4.h)
        L.qoq_kv4_cache_bytes.argtypes = [i64, i64, i64, i64]
        L.qoq_kv4_cache_bytes.restype = sz
        L.qoq_kv4_smooth_factors.argtypes = [vp, i64, i64, i64, vp, vp]
        L.qoq_kv4_smooth_factors.restype = ctypes.c_int
        L.qoq_kv4_append.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp, i64, vp]
        L.qoq_kv4_append.restype = ctypes.c_int
        L.qoq_kv4_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.qoq_kv4_attention_workspace_bytes.restype = sz
        L.qoq_kv4_decode_attention.argtypes = [vp, i64, i64, i64, i64, vp, vp, i64, vp, i64, vp,
                                               vp, sz, vp]
        L.qoq_kv4_decode_attention.restype = ctypes.c_int
        L.qoq_kv16_cache_bytes.argtypes = [i64, i64, i64, i64]
        L.qoq_kv16_cache_bytes.restype = sz
        L.qoq_kv16_append.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, i64, vp]
        L.qoq_kv16_append.restype = ctypes.c_int
        L.qoq_kv16_decode_attention.argtypes = [vp, i64, i64, i64, i64, vp, i64, vp, i64, vp, vp,
                                                sz, vp]
        L.qoq_kv16_decode_attention.restype = ctypes.c_int
        L.qoq_w4a16_weight_bytes.argtypes = [i64, i64]
        L.qoq_w4a16_weight_bytes.restype = sz
        L.qoq_w4a16_pack_weights.argtypes = [vp, i64, i64, vp, vp]
        L.qoq_w4a16_pack_weights.restype = ctypes.c_int
        L.qoq_w4a16_gemm.argtypes = [vp, i64, i64, vp, i64, vp, vp]
        L.qoq_w4a16_gemm.restype = ctypes.c_int
        L.qoq_stream_read.argtypes = [vp, sz, ctypes.c_int32, vp, vp]
        L.qoq_stream_read.restype = ctypes.c_int
        L.qoq_set_tuning.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
        L.qoq_set_tuning.restype = ctypes.c_int
        L.qoq_status_string.argtypes = [ctypes.c_int]
        L.qoq_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


# ---------------------------------------------------------------------------
# C-ABI mirrors (raw pointers as ints; stream as an int handle or None)
# ---------------------------------------------------------------------------
def qoq_status_string(status: int) -> str:
    return lib().qoq_status_string(int(status)).decode()


TUNING_KEYS = ("gemm", "variant", "kv4_splits", "kv4_paired")
_TUNING = {}


def set_tuning(key: str, value: Optional[str]) -> None:
    """Force a launch configuration (qoq_set_tuning; measurements and tests
    only): key in TUNING_KEYS, value None or "" to clear."""
    v = None if value in (None, "") else str(value)
    st = lib().qoq_set_tuning(key.encode(), None if v is None else v.encode())
    if st != 0:
        raise QoQError(st, "qoq_set_tuning")
    if v is None:
        _TUNING.pop(key, None)
    else:
        _TUNING[key] = v


def get_tuning(key: str) -> Optional[str]:
    """The value last set through set_tuning (None when unset)."""
    return _TUNING.get(key)


def clear_tuning() -> None:
    for k in TUNING_KEYS:
        set_tuning(k, None)


def qoq_stream_read(buf, nbytes: int, workgroups: int, sink, stream) -> int:
    """Measurement reference: one streaming read of `nbytes` at `buf`."""
    return lib().qoq_stream_read(buf, nbytes, workgroups, sink, stream)


def qoq_packed_weight_bytes(N: int, K: int, group: int = GROUP) -> int:
    return int(lib().qoq_packed_weight_bytes(N, K, group))


def qoq_act_bytes(M: int, K: int) -> int:
    return int(lib().qoq_act_bytes(M, K))


def qoq_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().qoq_gemm_workspace_bytes(M, N, K))


def qoq_pack_weights(W, N, K, group, packed, s1, canon, flags, stream) -> int:
    c = None
    if canon is not None:
        c = ctypes.byref(_Canonical(*canon))
    return lib().qoq_pack_weights(W, N, K, group, packed, s1, c, flags, stream)


def qoq_quantize_act(x, M, K, x8, s_x, stream) -> int:
    return lib().qoq_quantize_act(x, M, K, x8, s_x, stream)


def qoq_w4a8_gemm(x8, s_x, M, K, packed, s1, N, group, y, acc_debug, workspace,
                  workspace_bytes, stream) -> int:
    return lib().qoq_w4a8_gemm(x8, s_x, M, K, packed, s1, N, group, y, acc_debug, workspace,
                               workspace_bytes, stream)


def qoq_w4a8_gemm_noalloc(x8, s_x, M, K, packed, s1, N, group, y, acc_debug, stream) -> int:
    """qoq_w4a8_gemm with the library's fixed per-GPU scratch array in place
    of a workspace (nothing allocated; see include/qoq.h)."""
    return lib().qoq_w4a8_gemm_noalloc(x8, s_x, M, K, packed, s1, N, group, y, acc_debug,
                                       stream)


NOALLOC_SCRATCH_BYTES = 64 << 20   # QOQ_NOALLOC_SCRATCH_BYTES


def qoq_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().qoq_linear_workspace_bytes(M, N, K))


def qoq_linear_path(M: int, N: int, K: int) -> int:
    """1 one fused launch, 0 quantizer then GEMM, -1 invalid."""
    return int(lib().qoq_linear_path(M, N, K))


def qoq_w4a8_linear(x, M, K, packed, s1, N, group, y, acc_debug, workspace, workspace_bytes,
                    stream) -> int:
    return lib().qoq_w4a8_linear(x, M, K, packed, s1, N, group, y, acc_debug, workspace,
                                 workspace_bytes, stream)


# ---------------------------------------------------------------------------
# tensor-level helpers
# ---------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise QoQError(status, where)


def _need_gpu(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class PackedWeight:
    packed: torch.Tensor          # uint8 [qoq_packed_weight_bytes]
    s1: torch.Tensor              # float16 [N]
    N: int
    K: int
    group: int = GROUP
    q4: Optional[torch.Tensor] = None   # canonical outputs when requested
    s2: Optional[torch.Tensor] = None
    z: Optional[torch.Tensor] = None


def pack_weights(W: torch.Tensor, group: int = GROUP, canonical: bool = False) -> PackedWeight:
    """Quantize W fp32 [N, K] (device) in two levels and pack it."""
    _need_gpu(W, "W", torch.float32)
    N, K = W.shape
    nbytes = qoq_packed_weight_bytes(N, K, group)
    if nbytes == 0:
        raise QoQError(2, "qoq_pack_weights")
    dev = W.device
    packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    s1 = torch.empty(N, dtype=torch.float16, device=dev)
    canon = None
    q4 = s2 = z = None
    if canonical:
        q4 = torch.empty((N, K), dtype=torch.uint8, device=dev)
        s2 = torch.empty((N, K // group), dtype=torch.int8, device=dev)
        z = torch.empty((N, K // group), dtype=torch.uint8, device=dev)
        canon = (q4.data_ptr(), s2.data_ptr(), z.data_ptr())
    _check(qoq_pack_weights(W.data_ptr(), N, K, group, packed.data_ptr(), s1.data_ptr(), canon,
                            0, _stream(dev)), "qoq_pack_weights")
    return PackedWeight(packed, s1, N, K, group, q4, s2, z)


def pack_canonical(q4: torch.Tensor, s2: torch.Tensor, z: torch.Tensor, s1: torch.Tensor,
                   group: int = GROUP) -> PackedWeight:
    """Pack caller-supplied canonical codes (QOQ_PACK_FROM_CANONICAL)."""
    _need_gpu(q4, "q4", torch.uint8)
    _need_gpu(s2, "s2", torch.int8)
    _need_gpu(z, "z", torch.uint8)
    _need_gpu(s1, "s1", torch.float16)
    N, K = q4.shape
    nbytes = qoq_packed_weight_bytes(N, K, group)
    if nbytes == 0:
        raise QoQError(2, "qoq_pack_weights")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=q4.device)
    _check(qoq_pack_weights(None, N, K, group, packed.data_ptr(), None,
                            (q4.data_ptr(), s2.data_ptr(), z.data_ptr()), PACK_FROM_CANONICAL,
                            _stream(q4.device)), "qoq_pack_weights")
    return PackedWeight(packed, s1, N, K, group, q4, s2, z)


def empty_act(M: int, K: int, device) -> torch.Tensor:
    """An uninitialized x8 buffer for M tokens of K inputs (activation tile
    layout, shape (ceil(M/16), K/16, 16, 16))."""
    return torch.empty(((M + 15) // 16, K // 16, 16, 16), dtype=torch.int8, device=device)


def _check_act(x8: torch.Tensor, M: int, K: int):
    _need_gpu(x8, "x8", torch.int8)
    if tuple(x8.shape) != ((M + 15) // 16, K // 16, 16, 16):
        raise ValueError(f"x8 must have the activation tile shape {((M + 15) // 16, K // 16, 16, 16)}"
                         f" for M={M}, K={K}; got {tuple(x8.shape)}")


def quantize_act(x: torch.Tensor, out=None):
    """Per-token INT8 quantization of x fp16 [M, K] -> (x8 int8 in the
    activation tile layout, s_x fp32 [M])."""
    _need_gpu(x, "x", torch.float16)
    M, K = x.shape
    if out is None:
        x8 = empty_act(M, K, x.device)
        s_x = torch.empty(M, dtype=torch.float32, device=x.device)
    else:
        x8, s_x = out
        _check_act(x8, M, K)
        _need_gpu(s_x, "s_x", torch.float32)
        if s_x.shape != (M,):
            raise ValueError(f"s_x must have shape ({M},)")
    _check(qoq_quantize_act(x.data_ptr(), M, K, x8.data_ptr(), s_x.data_ptr(),
                            _stream(x.device)), "qoq_quantize_act")
    return x8, s_x


class Workspace:
    """A device buffer, grown on demand, for the workspace arguments of
    qoq_w4a8_gemm, qoq_w4a8_linear and the attention calls. One buffer
    serves any number of sequential calls on one stream; calls that may
    overlap (other streams) need a Workspace each.

    Growing never frees the buffer it replaces: the superseded buffers stay
    referenced (``retired``) for the Workspace's lifetime, so a HIP graph
    captured with an earlier, smaller buffer still writes into live memory
    when it is replayed after a later call has grown the workspace. Code
    that captures graphs should still pass a Workspace of its own, sized
    before the capture."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = torch.zeros(0, dtype=torch.uint8, device=self.device)
        self.retired = []

    def get(self, nbytes: int) -> torch.Tensor:
        if nbytes > self.buf.numel():
            if self.buf.numel():
                self.retired.append(self.buf)
            self.buf = torch.zeros(max(nbytes, 2 * self.buf.numel()), dtype=torch.uint8,
                                   device=self.device)
        return self.buf


_WORKSPACES = {}


def _default_workspace(device: torch.device) -> Workspace:
    """The default Workspace of (device, current stream): calls on different
    streams never share one."""
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, torch.cuda.current_stream(index).cuda_stream)
    if key not in _WORKSPACES:
        _WORKSPACES[key] = Workspace(torch.device("cuda", index))
    return _WORKSPACES[key]


def w4a8_gemm(x8: torch.Tensor, s_x: torch.Tensor, w: PackedWeight, acc_debug: bool = False,
              y: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None):
    """y fp16 [M, N] = fp16(acc * s_x * s1) for x8 / s_x from quantize_act
    (M = len(s_x)); also returns acc int32 if asked (acc_debug=True, or an
    int32 [M, N] tensor to write the accumulators into)."""
    _need_gpu(s_x, "s_x", torch.float32)
    if s_x.dim() != 1:
        raise ValueError("s_x must be 1-D [M]")
    M, K = s_x.shape[0], w.K
    _check_act(x8, M, K)
    dev = x8.device
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float16, device=dev)
    if isinstance(acc_debug, torch.Tensor):
        _need_gpu(acc_debug, "acc_debug", torch.int32)
        if tuple(acc_debug.shape) != (M, w.N):
            raise ValueError(f"acc_debug must have shape ({M}, {w.N})")
        acc = acc_debug
    else:
        acc = torch.empty((M, w.N), dtype=torch.int32, device=dev) if acc_debug else None
    if tuple(y.shape) != (M, w.N) or y.dtype != torch.float16:
        raise ValueError(f"y must be float16 of shape ({M}, {w.N})")
    ws_bytes = qoq_gemm_workspace_bytes(M, w.N, K) if M > 0 else 0
    ws_ptr = None
    if ws_bytes:
        ws = (workspace or _default_workspace(dev)).get(ws_bytes)
        ws_ptr = ws.data_ptr()
        ws_bytes = ws.numel()
    _check(qoq_w4a8_gemm(x8.data_ptr(), s_x.data_ptr(), M, K, w.packed.data_ptr(),
                         w.s1.data_ptr(), w.N, w.group, y.data_ptr(), _ptr(acc), ws_ptr,
                         ws_bytes, _stream(dev)), "qoq_w4a8_gemm")
    return (y, acc) if acc is not None else y


def w4a8_linear(x: torch.Tensor, w: PackedWeight, acc_debug: bool = False,
                y: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None):
    """y fp16 [M, N] from fp16 activations x [M, K] in one call: per-token
    quantization and the W4A8 GEMM (one fused launch for small M, otherwise
    the quantizer into the workspace and the GEMM); also returns acc int32
    if asked."""
    _need_gpu(x, "x", torch.float16)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, weights have K={w.K}")
    dev = x.device
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float16, device=dev)
    acc = torch.empty((M, w.N), dtype=torch.int32, device=dev) if acc_debug else None
    ws_bytes = qoq_linear_workspace_bytes(M, w.N, K) if M > 0 else 0
    ws_ptr = None
    if ws_bytes:
        ws = (workspace or _default_workspace(dev)).get(ws_bytes)
        ws_ptr = ws.data_ptr()
        ws_bytes = ws.numel()
    _check(qoq_w4a8_linear(x.data_ptr(), M, K, w.packed.data_ptr(), w.s1.data_ptr(), w.N,
                           w.group, y.data_ptr(), _ptr(acc), ws_ptr, ws_bytes, _stream(dev)),
           "qoq_w4a8_linear")
    return (y, acc) if acc_debug else y


# ---------------------------------------------------------------------------
# comparison GEMMs (W8A8 per-channel; W4A4 per-group with partial-sum
# scaling; W4A16 weight-only with fp16 dequantization)
# ---------------------------------------------------------------------------
def w8a8_pack_weights(W: torch.Tensor):
    """Per-channel INT8 weights of W fp32 [N, K] -> (packed uint8, s fp16 [N])."""
    _need_gpu(W, "W", torch.float32)
    N, K = W.shape
    nbytes = int(lib().qoq_w8a8_weight_bytes(N, K))
    if nbytes == 0:
        raise QoQError(2, "qoq_w8a8_pack_weights")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    s = torch.empty(N, dtype=torch.float16, device=W.device)
    _check(lib().qoq_w8a8_pack_weights(W.data_ptr(), N, K, packed.data_ptr(), s.data_ptr(),
                                       _stream(W.device)), "qoq_w8a8_pack_weights")
    return packed, s


def w8a8_gemm(x8: torch.Tensor, s_x: torch.Tensor, packed: torch.Tensor, s: torch.Tensor,
              N: int, acc_debug: bool = False):
    """W8A8 GEMM on x8/s_x from quantize_act: y fp16 [M, N] (and acc int32)."""
    _need_gpu(s_x, "s_x", torch.float32)
    M, K = s_x.shape[0], x8.shape[1] * 16
    _check_act(x8, M, K)
    dev = x8.device
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if acc_debug else None
    _check(lib().qoq_w8a8_gemm(x8.data_ptr(), s_x.data_ptr(), M, K, packed.data_ptr(),
                               s.data_ptr(), N, y.data_ptr(), _ptr(acc), _stream(dev)),
           "qoq_w8a8_gemm")
    return (y, acc) if acc_debug else y


def w4a4_pack_weights(W: torch.Tensor) -> torch.Tensor:
    """Per-(channel, group) INT4 weights of W fp32 [N, K] -> packed uint8."""
    _need_gpu(W, "W", torch.float32)
    N, K = W.shape
    nbytes = int(lib().qoq_w4a4_weight_bytes(N, K))
    if nbytes == 0:
        raise QoQError(2, "qoq_w4a4_pack_weights")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    _check(lib().qoq_w4a4_pack_weights(W.data_ptr(), N, K, packed.data_ptr(), _stream(W.device)),
           "qoq_w4a4_pack_weights")
    return packed


def w4a4_quantize_act(x: torch.Tensor) -> torch.Tensor:
    """Per-(token, group) INT4 activations of x fp16 [M, K] -> act uint8
    (x4 tile layout, then the fp32 group scales)."""
    _need_gpu(x, "x", torch.float16)
    M, K = x.shape
    nbytes = int(lib().qoq_w4a4_act_bytes(M, K)) if M > 0 else 0
    act = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check(lib().qoq_w4a4_quantize_act(x.data_ptr(), M, K, act.data_ptr(), _stream(x.device)),
           "qoq_w4a4_quantize_act")
    return act


def w4a4_gemm(act: torch.Tensor, M: int, K: int, packed: torch.Tensor, N: int) -> torch.Tensor:
    """W4A4 GEMM with per-group partial-sum scaling: y fp16 [M, N]."""
    _need_gpu(act, "act", torch.uint8)
    y = torch.empty((M, N), dtype=torch.float16, device=act.device)
    _check(lib().qoq_w4a4_gemm(act.data_ptr(), M, K, packed.data_ptr(), N, y.data_ptr(),
                               _stream(act.device)), "qoq_w4a4_gemm")
    return y


def w4a16_pack_weights(W: torch.Tensor) -> torch.Tensor:
    """Per-(channel, group) UINT4 weights with fp16 scale and zero of W fp32
    [N, K] -> packed uint8."""
    _need_gpu(W, "W", torch.float32)
    N, K = W.shape
    nbytes = int(lib().qoq_w4a16_weight_bytes(N, K))
    if nbytes == 0:
        raise QoQError(2, "qoq_w4a16_pack_weights")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    _check(lib().qoq_w4a16_pack_weights(W.data_ptr(), N, K, packed.data_ptr(), _stream(W.device)),
           "qoq_w4a16_pack_weights")
    return packed


def w4a16_gemm(x: torch.Tensor, packed: torch.Tensor, N: int) -> torch.Tensor:
    """W4A16 GEMM on fp16 x [M, K]: weights dequantized to fp16 in the main
    loop, fp32 accumulation, y fp16 [M, N]."""
    _need_gpu(x, "x", torch.float16)
    _need_gpu(packed, "packed", torch.uint8)
    M, K = x.shape
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check(lib().qoq_w4a16_gemm(x.data_ptr(), M, K, packed.data_ptr(), N, y.data_ptr(),
                                _stream(x.device)), "qoq_w4a16_gemm")
    return y


# ---------------------------------------------------------------------------
# KV4 decode attention with SmoothAttention scaling
# ---------------------------------------------------------------------------
KV4_HEAD_DIM = 128


def kv4_cache_bytes(B: int, H_kv: int, capacity: int) -> int:
    return int(lib().qoq_kv4_cache_bytes(B, H_kv, capacity, KV4_HEAD_DIM))


def kv4_alloc_cache(B: int, H_kv: int, capacity: int, device) -> torch.Tensor:
    """Device buffer for a KV4 cache (contents undefined until appended)."""
    nbytes = kv4_cache_bytes(B, H_kv, capacity)
    if nbytes == 0:
        raise QoQError(2, "qoq_kv4_cache_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kv4_smooth_factors(k_calib: torch.Tensor) -> torch.Tensor:
    """lambda [H_kv, D] fp16 from calibration keys [..., H_kv, D] fp16."""
    _need_gpu(k_calib, "k_calib", torch.float16)
    H_kv, D = k_calib.shape[-2:]
    T = k_calib.numel() // (H_kv * D)
    lam = torch.empty((H_kv, D), dtype=torch.float16, device=k_calib.device)
    _check(lib().qoq_kv4_smooth_factors(k_calib.data_ptr(), T, H_kv, D, lam.data_ptr(),
                                        _stream(k_calib.device)), "qoq_kv4_smooth_factors")
    return lam


def kv4_append(k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor, start: torch.Tensor,
               cache: torch.Tensor, capacity: int) -> None:
    """Append k, v [B, T_new, H_kv, D] fp16 at positions start[b] (device int32)."""
    _need_gpu(k, "k", torch.float16)
    _need_gpu(v, "v", torch.float16)
    _need_gpu(lam, "lambda", torch.float16)
    _need_gpu(start, "start", torch.int32)
    _need_gpu(cache, "cache", torch.uint8)
    if k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must both be [B, T_new, H_kv, D]")
    B, T, H_kv, D = k.shape
    _check(lib().qoq_kv4_append(k.data_ptr(), v.data_ptr(), B, T, H_kv, D, lam.data_ptr(),
                                start.data_ptr(), cache.data_ptr(), capacity, _stream(k.device)),
           "qoq_kv4_append")


def kv4_decode_attention(q: torch.Tensor, lam: torch.Tensor, cache: torch.Tensor, capacity: int,
                         lens: torch.Tensor, max_len: int, H_kv: int,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[Workspace] = None) -> torch.Tensor:
    """out [B, H, D] fp16 = softmax(q~ k^T / sqrt(D)) v over the KV4 cache."""
    _need_gpu(q, "q", torch.float16)
    _need_gpu(lam, "lambda", torch.float16)
    _need_gpu(cache, "cache", torch.uint8)
    _need_gpu(lens, "lens", torch.int32)
    B, H, D = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float16, device=dev)
    wsb = int(lib().qoq_kv4_attention_workspace_bytes(B, H, H_kv, D, max_len))
    ws_ptr = None
    if wsb:
        ws = (workspace or _default_workspace(dev)).get(wsb)
        ws_ptr, wsb = ws.data_ptr(), ws.numel()
    _check(lib().qoq_kv4_decode_attention(q.data_ptr(), B, H, H_kv, D, lam.data_ptr(),
                                          cache.data_ptr(), capacity, lens.data_ptr(), max_len,
                                          out.data_ptr(), ws_ptr, wsb, _stream(dev)),
           "qoq_kv4_decode_attention")
    return out


def kv16_alloc_cache(B: int, H_kv: int, capacity: int, device) -> torch.Tensor:
    """Device buffer for the fp16 comparison cache."""
    nbytes = int(lib().qoq_kv16_cache_bytes(B, H_kv, capacity, KV4_HEAD_DIM))
    if nbytes == 0:
        raise QoQError(2, "qoq_kv16_cache_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kv16_append(k: torch.Tensor, v: torch.Tensor, start: torch.Tensor, cache: torch.Tensor,
                capacity: int) -> None:
    _need_gpu(k, "k", torch.float16)
    _need_gpu(v, "v", torch.float16)
    _need_gpu(start, "start", torch.int32)
    _need_gpu(cache, "cache", torch.uint8)
    if k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must both be [B, T_new, H_kv, D]")
    B, T, H_kv, D = k.shape
    _check(lib().qoq_kv16_append(k.data_ptr(), v.data_ptr(), B, T, H_kv, D, start.data_ptr(),
                                 cache.data_ptr(), capacity, _stream(k.device)), "qoq_kv16_append")


def kv16_decode_attention(q: torch.Tensor, cache: torch.Tensor, capacity: int, lens: torch.Tensor,
                          max_len: int, H_kv: int, out: Optional[torch.Tensor] = None,
                          workspace: Optional[Workspace] = None) -> torch.Tensor:
    """out [B, H, D] fp16 = softmax(q k^T / sqrt(D)) v over the fp16 cache."""
    _need_gpu(q, "q", torch.float16)
    _need_gpu(cache, "cache", torch.uint8)
    _need_gpu(lens, "lens", torch.int32)
    B, H, D = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float16, device=dev)
    wsb = int(lib().qoq_kv4_attention_workspace_bytes(B, H, H_kv, D, max_len))
    ws_ptr = None
    if wsb:
        ws = (workspace or _default_workspace(dev)).get(wsb)
        ws_ptr, wsb = ws.data_ptr(), ws.numel()
    _check(lib().qoq_kv16_decode_attention(q.data_ptr(), B, H, H_kv, D, cache.data_ptr(), capacity,
                                           lens.data_ptr(), max_len, out.data_ptr(), ws_ptr, wsb,
                                           _stream(dev)), "qoq_kv16_decode_attention")
    return out
