"""Guard bands for the GPU tests: an output buffer placed inside a larger
allocation whose bytes before and after it hold a known pattern, checked on
the host after the call.  A kernel writing even one byte outside its output
(an off-by-one slice offset, a tail tile running past the end, a peer copy
into the wrong place) changes the pattern, which comparing the output itself
cannot see."""
import torch

GUARD = 4096          # bytes of pattern on each side
PATTERN = 0xA5


class Guarded:
    """n elements of `dtype`, `offset` bytes past a 4096-byte boundary of the
    allocation (a multiple of the element size; not a multiple of 16 puts the
    buffer off the 16-byte grid), on `device` (pinned when on the host)."""

    def __init__(self, n, dtype, offset=0, device="cuda", init=None):
        es = torch.empty(0, dtype=dtype).element_size()
        if offset % es:
            raise ValueError("offset must be a multiple of the element size")
        self.n, self.es, self.offset = n, es, offset
        self.lo = GUARD + offset
        self.hi = self.lo + n * es
        total = self.hi + GUARD
        pin = device == "cpu" and torch.cuda.is_available()
        self.backing = torch.full((total,), PATTERN, dtype=torch.uint8, device=device, pin_memory=pin)
        self.t = self.backing[self.lo:self.hi].view(dtype)
        if init is not None:
            self.t.copy_(init.reshape(-1))

    def check(self, what):
        torch.cuda.synchronize()
        for name, band in (("before", self.backing[:self.lo]), ("after", self.backing[self.hi:])):
            b = band.cpu()
            bad = torch.nonzero(b != PATTERN)
            assert bad.numel() == 0, "%s: %d guard bytes %s the buffer changed (first at %d of %d)" % (
                what, bad.numel(), name, int(bad[0]), b.numel())
