"""Torch conveniences over the C ABI: torch supplies device memory, pinned
host memory and streams; every step of the path runs in libtb.

    RotatedSources   K slices per source (PR #365 rotation), prepared with
                     tb_prep_reference + tb_prep_sources
    reduce_copy      tb_reduce_copy on tensors / raw device addresses
    make_desc        (src_off, dst_off, bytes) offsets -> device tb_copy_desc array
    batched_copy     tb_batched_copy on a device descriptor tensor
    DescRing         tb_ring_* (descriptor-slot ring) over host descriptor arrays
"""
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import _tb


def stream_handle(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _addr(x) -> int:
    return int(x.data_ptr()) if isinstance(x, torch.Tensor) else int(x)


def host_reference(nfloats: int, buffer_idx: int, fill=None, pin: bool = True) -> torch.Tensor:
    """PrepareReference of one source into a (pinned) host float32 tensor."""
    t = torch.empty(nfloats, dtype=torch.float32, pin_memory=pin and torch.cuda.is_available())
    if nfloats:
        _tb.tb_prep_reference(t.data_ptr(), nfloats, buffer_idx, fill)
    return t


class RotatedSources:
    """nsrc sources of nfloats floats, each replicated into K slices."""

    def __init__(self, nsrc: int, nfloats: int, rotate_bytes: int, fill=None,
                 device: Optional[torch.device] = None, host_refs: Optional[Sequence[torch.Tensor]] = None,
                 stream: Optional[torch.cuda.Stream] = None):
        self.nsrc = nsrc
        self.nfloats = nfloats
        self.num_bytes = nfloats * 4
        self.k = _tb.tb_num_slices(self.num_bytes, rotate_bytes)
        self.stride = _tb.tb_slice_stride(self.num_bytes)
        dev = device or torch.device("cuda", torch.cuda.current_device())
        self.buffers: List[torch.Tensor] = [
            torch.empty(max(1, self.k * self.stride), dtype=torch.uint8, device=dev) for _ in range(nsrc)]
        sh = stream_handle(stream)
        self.host_refs = list(host_refs) if host_refs is not None else [
            host_reference(nfloats, b, fill) for b in range(nsrc)]
        for b in range(nsrc):
            _tb.tb_prep_sources(self.buffers[b].data_ptr(), self.stride, self.k,
                                self.host_refs[b].data_ptr(), nfloats, sh)

    @property
    def bases(self) -> List[int]:
        return [int(b.data_ptr()) for b in self.buffers]

    def pointers(self, iteration: int) -> List[int]:
        """Device addresses of the slices iteration `iteration` reads (untimed host arithmetic)."""
        return _tb.tb_rotate_sources(self.bases, self.stride, self.k, iteration)

    def slice_view(self, b: int, s: int) -> torch.Tensor:
        """Source b, slice s, as a float32 tensor view."""
        off = s * self.stride
        return self.buffers[b][off:off + self.num_bytes].view(torch.float32)


def reduce_copy(dst, srcs, nfloats: Optional[int] = None, stream: Optional[torch.cuda.Stream] = None,
                memset_byte: int = 0) -> None:
    """dst = srcs[0] + ... (fixed order) via tb_reduce_copy; tensors or device addresses."""
    if isinstance(dst, torch.Tensor):
        if dst.dtype != torch.float32 or not dst.is_cuda or not dst.is_contiguous():
            raise ValueError("dst must be a contiguous float32 CUDA tensor")
        if nfloats is None:
            nfloats = dst.numel()
        elif nfloats > dst.numel():
            raise ValueError("nfloats exceeds dst")
    elif nfloats is None:
        raise ValueError("nfloats is required with raw addresses")
    for s in srcs:
        if isinstance(s, torch.Tensor) and (s.dtype != torch.float32 or not s.is_cuda or not s.is_contiguous()
                                            or s.numel() < nfloats):
            raise ValueError("sources must be contiguous float32 CUDA tensors of at least nfloats elements")
    _tb.tb_reduce_copy(_addr(dst), [_addr(s) for s in srcs], nfloats, stream_handle(stream), memset_byte)


def make_desc(offsets: np.ndarray, src_base: int, dst_base: int, device=None) -> torch.Tensor:
    """Device int64 tensor (n, 3) of tb_copy_desc records from (src_off, dst_off, bytes) offsets."""
    o = np.ascontiguousarray(offsets, dtype=np.uint64).reshape(-1, 3)
    d = o.copy()
    d[:, 0] += np.uint64(src_base)
    d[:, 1] += np.uint64(dst_base)
    dev = device or torch.device("cuda", torch.cuda.current_device())
    return torch.from_numpy(d.view(np.int64)).to(dev)


def batched_copy(desc: torch.Tensor, ncopies: Optional[int] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> None:
    """tb_batched_copy over a device (n, 3) int64 descriptor tensor."""
    if (desc.dtype != torch.int64 or not desc.is_cuda or not desc.is_contiguous() or desc.dim() != 2
            or desc.shape[1] != 3):
        raise ValueError("desc must be a contiguous int64 CUDA tensor of shape (n, 3)")
    n = desc.shape[0] if ncopies is None else ncopies
    if not 0 <= n <= desc.shape[0]:
        raise ValueError("ncopies must be between 0 and the number of descriptors in desc")
    _tb.tb_batched_copy(desc.data_ptr(), n, stream_handle(stream))


class DescRing:
    """Descriptor-slot ring on the current device: submit host (n, 3) uint64
    descriptor arrays (absolute src, dst, bytes) and poll their tickets.
    direct: the kernel reads the pinned slots itself (faster in every measured
    case); otherwise each slot is first copied to device memory."""

    def __init__(self, nslots: int = 32, slot_descs: int = 8192, direct: bool = True,
                 stream: Optional[torch.cuda.Stream] = None):
        self.handle = _tb.tb_ring_create(nslots, slot_descs, _tb.TB_RING_DIRECT if direct else _tb.TB_RING_STAGED,
                                         stream_handle(stream))

    def submit(self, desc: np.ndarray) -> int:
        d = np.ascontiguousarray(desc, dtype=np.uint64).reshape(-1, 3)
        return _tb.tb_ring_submit(self.handle, d.ctypes.data, d.shape[0])

    def poll(self, ticket: int) -> bool:
        return _tb.tb_ring_poll(self.handle, ticket)

    def wait(self, ticket: int) -> None:
        _tb.tb_ring_wait(self.handle, ticket)

    def close(self) -> None:
        if self.handle:
            h, self.handle = self.handle, 0
            _tb.tb_ring_destroy(h)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
