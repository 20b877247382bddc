"""Helpers for the GPU parity tests: moving BF16 bit patterns and codes
between NumPy and device tensors, and guard-banded output buffers that catch
stray writes."""
import sys

import numpy as np

CANARY = 0xA5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bf16_f64(t) -> np.ndarray:
    """Device BF16 tensor -> exact float64 values."""
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Guarded:
    """A 2-D device buffer [rows, cols] of `dtype` inside a larger byte buffer
    whose guard bands (before, after, and the row padding when ld > cols) are
    filled with a canary byte.  `view` is what the kernel writes."""

    def __init__(self, rows, cols, dtype, ld=None, guard_bytes=4096):
        import torch
        esz = torch.empty(0, dtype=dtype).element_size()
        ld = cols if ld is None else ld
        self.rows, self.cols, self.ld, self.esz = rows, cols, ld, esz
        self.g = guard_bytes
        body = rows * ld * esz
        self.raw = torch.full((guard_bytes * 2 + body,), CANARY, dtype=torch.uint8, device="cuda")
        inner = self.raw[guard_bytes:guard_bytes + body].view(dtype)
        self.view = inner.view(rows, ld)[:, :cols] if rows else inner.view(0, cols)

    def check_canaries(self):
        raw = self.raw.cpu().numpy()
        g = self.g
        assert np.all(raw[:g] == CANARY), "write before the buffer"
        assert np.all(raw[len(raw) - g:] == CANARY), "write after the buffer"
        if self.ld > self.cols and self.rows:
            body = raw[g:len(raw) - g].reshape(self.rows, self.ld * self.esz)
            assert np.all(body[:, self.cols * self.esz:] == CANARY), "write into row padding"
