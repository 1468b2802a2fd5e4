"""Guard bands for GPU outputs: a buffer is allocated with GUARD sentinel bytes
before and after the region a call may write, and the bands are checked after
the call, so a kernel that writes past either end of its output (or workspace)
fails the test that ran it."""
import math

import torch

GUARD = 4096          # bytes on each side; keeps the region 4 KiB aligned
SENTINEL = 0xA5


def alloc(shape, dtype, device, fill=SENTINEL):
    """(buffer, view): `view` of `shape`/`dtype` inside a byte buffer whose
    guard bands (and, until the call overwrites it, the view) hold `fill`."""
    shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
    nbytes = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((GUARD + nbytes + GUARD,), fill, dtype=torch.uint8, device=device)
    view = buf[GUARD:GUARD + nbytes].view(dtype).view(shape)
    return buf, view


def check(buf, what="output"):
    """Raise if a byte of either guard band changed."""
    head = buf[:GUARD].cpu()
    tail = buf[buf.numel() - GUARD:].cpu()
    bad_head = int((head != SENTINEL).sum())
    bad_tail = int((tail != SENTINEL).sum())
    if bad_head or bad_tail:
        raise AssertionError(f"{what}: {bad_head} bytes before and {bad_tail} bytes after "
                             f"the buffer were overwritten")
