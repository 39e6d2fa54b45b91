"""Helpers for the GPU parity tests: device buffers with guard bands, uploads."""

import sys

import numpy as np
import torch

GUARD = 4096          # bytes of canary before and after every output buffer
CANARY = 0xA5


def say(msg):
    """Name the case on stdout before a GPU step (survives a lost box)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def upload_bits(bits):
    """numpy unsigned array -> device tensor of the same bytes (int view)."""
    bits = np.ascontiguousarray(bits)
    view = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[bits.dtype.itemsize]
    t = torch.from_numpy(bits.view(view) if view is not np.uint8 else bits)
    return t.to(device())


def upload_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device())


class Guarded:
    """A device output buffer of `nbytes` framed by canary bytes."""

    def __init__(self, nbytes, fill=None):
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device=device())
        if fill is not None:
            fb = np.ascontiguousarray(fill).view(np.uint8).reshape(-1)
            assert fb.size == nbytes
            self.raw[GUARD:GUARD + nbytes] = torch.from_numpy(fb).to(device())

    @property
    def ptr(self):
        return self.raw.data_ptr() + GUARD

    def host(self, dtype):
        b = self.raw[GUARD:GUARD + self.nbytes].cpu().numpy()
        return b.view(dtype)

    def guards_intact(self):
        g = torch.cat([self.raw[:GUARD], self.raw[GUARD + self.nbytes:]])
        return bool((g == CANARY).all().item())
