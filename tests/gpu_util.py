"""Helpers for the GPU parity tests: host<->device copies of numpy arrays
and guard-banded output buffers."""
import numpy as np
import pytest
import torch

GUARD = 256          # canary bytes on each side of an output buffer
CANARY = 0xA5


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_amd as m   # raises if the library is missing
    return m


def dev_bf16(bits):
    """numpy uint16 bf16 bit patterns -> cuda bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def dev_i64(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int64)).cuda()


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.contiguous().cpu().numpy()


class Guarded:
    """A device byte buffer with canary bands around the payload.

    view(dtype, shape) is the payload; check() asserts the bands are intact."""

    def __init__(self, nbytes, align=256):
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.off = GUARD

    def view(self, dtype, shape):
        t = self.raw[self.off:self.off + self.nbytes].view(dtype)
        return t.view(shape)

    def check(self):
        r = self.raw.cpu().numpy()
        assert np.all(r[:GUARD] == CANARY) and np.all(r[GUARD + self.nbytes:] == CANARY), \
            "write outside the output buffer"
