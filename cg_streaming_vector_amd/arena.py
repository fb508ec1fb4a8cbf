"""One HBM allocation carved into 2 MB-aligned arrays.

The streaming kernels run several arrays in lockstep (the fused CG update
reads four and writes two at the same index). On MI355X their throughput
depends on where those arrays sit relative to each other: packed back to back
in one allocation at 2 MB granularity, the six streams of the fused update
sustain about 5 % more bandwidth than the same arrays at scattered offsets,
and some odd relative offsets cost over 10 %. An Arena is one device
allocation from which a workload's arrays are taken in order, each starting
on a 2 MB boundary of the allocation.
"""
from __future__ import annotations

ALIGN = 2 << 20


class Arena:
    def __init__(self, nbytes: int, device, align: int = ALIGN):
        import torch
        self.align = align
        self.buf = torch.empty(int(nbytes) + align, dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        self.pos = (-base) % align  # first aligned offset inside the buffer
        self.cap = self.pos + int(nbytes)

    @staticmethod
    def slot(nbytes: int, align: int = ALIGN) -> int:
        """Bytes an array of nbytes occupies in an arena."""
        return (int(nbytes) + align - 1) // align * align

    def empty(self, n: int, dtype, pad: int = 0):
        """An uninitialised 1-D tensor of n elements at the next aligned slot;
        `pad` more granules of `align` bytes are left unused after it (so that
        arrays whose sizes are powers of two do not sit a power of two
        apart)."""
        import torch
        itemsize = torch.empty(0, dtype=dtype).element_size()
        nbytes = int(n) * itemsize
        if self.pos + nbytes > self.cap:
            raise MemoryError("arena exhausted")
        t = self.buf[self.pos:self.pos + nbytes].view(dtype)
        self.pos += self.slot(max(nbytes, 1), self.align) + int(pad) * self.align
        return t

    def put(self, src):
        """A copy of tensor src (any device) in the arena, of the same shape."""
        t = self.empty(src.numel(), src.dtype)
        t.copy_(src.reshape(-1))
        return t.view(src.shape)
