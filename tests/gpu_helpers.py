"""Helpers for GPU parity tests: raw byte transfers and guarded output buffers."""
import numpy as np
import torch

GUARD = 256          # bytes of canary before and after each output buffer
CANARY = 0xA5


def dev(a):
    """numpy raw array -> cuda tensor with the same bytes (16-bit floats travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def host(t, np_dtype):
    return t.cpu().numpy().view(np_dtype)


class Guarded:
    """An output buffer with canary bytes on both sides; .t is the tensor the library writes."""

    def __init__(self, shape, torch_dtype, fill=None):
        es = torch.empty((), dtype=torch_dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        nbytes = n * es
        self.raw = torch.full((GUARD + nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.nbytes = nbytes
        self.t = self.raw[GUARD:GUARD + nbytes].view(torch_dtype).view(*shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self):
        r = self.raw.cpu().numpy()
        assert (r[:GUARD] == CANARY).all(), "write before the start of the output buffer"
        assert (r[GUARD + self.nbytes:] == CANARY).all(), "write past the end of the output buffer"


def sync():
    torch.cuda.synchronize()
