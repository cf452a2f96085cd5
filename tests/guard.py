"""Guard bands for GPU output buffers: every buffer a kernel writes is
carved out of a larger allocation whose bytes before and after it hold a
known pattern; after the launch the pattern must be intact, so a store out
of bounds on either side fails the test instead of passing unseen."""
import numpy as np
import torch

PAD = 256            # bytes on each side (keeps the inner buffer 256-byte aligned)
PATTERN = 0xA5


class Guarded:
    def __init__(self, shape, dtype, device, fill=None):
        itemsize = torch.empty(0, dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * itemsize
        self.raw = torch.full((self.nbytes + 2 * PAD,), PATTERN, dtype=torch.uint8, device=device)
        inner = self.raw[PAD:PAD + self.nbytes]
        if fill is not None:
            inner.fill_(fill)
        self.t = inner.view(dtype).view(shape)

    def check(self, what="buffer"):
        torch.cuda.synchronize()
        lo = self.raw[:PAD]
        hi = self.raw[PAD + self.nbytes:]
        assert bool((lo == PATTERN).all()), f"{what}: bytes before the buffer were overwritten"
        assert bool((hi == PATTERN).all()), f"{what}: bytes after the buffer were overwritten"


class GuardedWorkspace:
    """A Workspace stand-in whose buffer has guard bands (fixed capacity)."""

    def __init__(self, nbytes, device):
        self.g = Guarded((max(int(nbytes), 16),), torch.uint8, device)
        self.buf = self.g.t

    def get(self, nbytes):
        assert nbytes <= self.buf.numel(), "guarded workspace too small"
        return self.buf

    def check(self):
        self.g.check("workspace")
