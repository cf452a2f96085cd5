"""The streaming-read measurement reference reads every 16-byte word of its
buffer: a single word equal to the kernel's sentinel, anywhere in the
buffer, reaches the sink; an all-zero buffer leaves it untouched."""
import pytest
import torch

import bit_integer_gemm_amd as qoq  # noqa: E402  (a broken binding must fail, not skip)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 0x9E3779B9


def _read(buf, workgroups):
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    st = qoq.qoq_stream_read(buf.data_ptr(), buf.numel() * 4, workgroups, sink.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("words", [4, 4 * 1000, 4 * 262147])
@pytest.mark.parametrize("workgroups", [0, 1, 7, 256])
def test_every_word_is_read(words, workgroups):
    print(f"\n[gpu-case] stream_read words={words} wg={workgroups}", flush=True)
    buf = torch.zeros(words, dtype=torch.int32, device=DEV)
    assert _read(buf, workgroups) == 0
    for pos in sorted({0, words // 2 + 1, words - 1}):
        buf.zero_()
        buf[pos] = SENTINEL - (1 << 32)      # the int32 bit pattern of the sentinel
        assert _read(buf, workgroups) == SENTINEL, pos
