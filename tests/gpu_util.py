"""Helpers for the GPU parity tests: device buffers at chosen byte offsets with
guard bands, and a loud failure when no GPU or no HIP library is present."""
import sys

import numpy as np
import pytest

GUARD = 256          # guard bytes on each side of a tested buffer
GUARD_BYTE = 0xEE


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a lost box still says what ran."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU: the HIP path has no CPU fallback")
    import copy_reduce_amd  # noqa: F401  (raises if libtb.so is missing)
    return torch


class DevBuf:
    """`nbytes` of device memory at `offset` bytes past a 256-aligned base,
    surrounded by GUARD bytes of GUARD_BYTE."""

    def __init__(self, torch, nbytes: int, offset: int = 0, fill: int = GUARD_BYTE):
        self.nbytes, self.offset = nbytes, offset
        self.t = torch.full((GUARD + offset + nbytes + GUARD,), fill, dtype=torch.uint8, device="cuda")
        self.start = GUARD + offset
        if fill != GUARD_BYTE:
            self.t[:self.start] = GUARD_BYTE
            self.t[self.start + nbytes:] = GUARD_BYTE

    @property
    def ptr(self) -> int:
        return int(self.t.data_ptr()) + self.start

    def upload(self, arr: np.ndarray):
        import torch
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert b.size == self.nbytes
        if b.size:
            self.t[self.start:self.start + b.size].copy_(torch.from_numpy(b.copy()))
        return self

    def download(self) -> np.ndarray:
        return self.t[self.start:self.start + self.nbytes].cpu().numpy()

    def guards_intact(self) -> bool:
        full = self.t.cpu().numpy()
        return bool(np.all(full[:self.start] == GUARD_BYTE) and np.all(full[self.start + self.nbytes:] == GUARD_BYTE))
