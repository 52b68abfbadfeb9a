"""ctypes binding of libtb_roofs.so (include/tb_roofs.h): the measuring
instruments of bench.py --roofs, with the names of their C calls, plus the
host-side cut of a batch of copies into tiles of at most 4 KiB.

Loaded only by whoever measures: the transfer path itself never uses it.
"""
import ctypes
import os

import numpy as np

from ._tb import PKG

ROOFS_LIB_PATH = os.path.join(PKG, "libtb_roofs.so")

TBR_OK, TBR_ERR_INVALID, TBR_ERR_HIP = 0, -1, -2
TBR_STORE_DEVICE, TBR_STORE_STREAMING, TBR_STORE_NT = 0, 1, 2
TBR_MAX_BUFS = 17
TILE_BYTES = 4096

EXPORTS = ("tbr_read", "tbr_write", "tbr_copy", "tbr_combine", "tbr_tiles_copy", "tbr_tiles_write",
           "tbr_tiles_read", "tbr_last_hip_error")

if not os.path.exists(ROOFS_LIB_PATH):
    raise ImportError(f"{ROOFS_LIB_PATH} is missing: build the HIP libraries first "
                      "(python -c 'import __graft_entry__ as g; g.build()')")

lib = ctypes.CDLL(ROOFS_LIB_PATH)
_u64, _u32, _i32, _vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p
_SIGS = {
    "tbr_read": (ctypes.c_int, [_vp, _i32, _u64, _vp]),
    "tbr_write": (ctypes.c_int, [_vp, _i32, _u64, _u32, _u32, _vp]),
    "tbr_copy": (ctypes.c_int, [_vp, _vp, _u64, _u32, _vp]),
    "tbr_combine": (ctypes.c_int, [_vp, _i32, _vp, _u64, _u32, _vp]),
    "tbr_tiles_copy": (ctypes.c_int, [_vp, _u32, _u32, _vp]),
    "tbr_tiles_write": (ctypes.c_int, [_vp, _u32, _u32, _u32, _vp]),
    "tbr_tiles_read": (ctypes.c_int, [_vp, _u32, _vp]),
    "tbr_last_hip_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class RoofError(RuntimeError):
    pass


def _check(fn, status):
    if status != TBR_OK:
        msg = "invalid argument" if status == TBR_ERR_INVALID else "HIP error: " + lib.tbr_last_hip_error().decode()
        raise RoofError(f"{fn} failed with {status} ({msg})")


def _ptrs(ptrs):
    return (ctypes.c_void_p * max(1, len(ptrs)))(*[int(p) for p in ptrs])


def tbr_read(buf_ptrs, bytes_each: int, stream: int) -> None:
    _check("tbr_read", lib.tbr_read(_ptrs(buf_ptrs), len(buf_ptrs), bytes_each, stream))


def tbr_write(buf_ptrs, bytes_each: int, word: int, policy: int, stream: int) -> None:
    _check("tbr_write", lib.tbr_write(_ptrs(buf_ptrs), len(buf_ptrs), bytes_each, word, policy, stream))


def tbr_copy(dst_ptr: int, src_ptr: int, nbytes: int, policy: int, stream: int) -> None:
    _check("tbr_copy", lib.tbr_copy(dst_ptr, src_ptr, nbytes, policy, stream))


def tbr_combine(src_ptrs, dst_ptr: int, bytes_each: int, policy: int, stream: int) -> None:
    _check("tbr_combine", lib.tbr_combine(_ptrs(src_ptrs), len(src_ptrs), dst_ptr, bytes_each, policy, stream))


def tbr_tiles_copy(tiles_dev_ptr: int, ntiles: int, policy: int, stream: int) -> None:
    _check("tbr_tiles_copy", lib.tbr_tiles_copy(tiles_dev_ptr, ntiles, policy, stream))


def tbr_tiles_write(tiles_dev_ptr: int, ntiles: int, word: int, policy: int, stream: int) -> None:
    _check("tbr_tiles_write", lib.tbr_tiles_write(tiles_dev_ptr, ntiles, word, policy, stream))


def tbr_tiles_read(tiles_dev_ptr: int, ntiles: int, stream: int) -> None:
    _check("tbr_tiles_read", lib.tbr_tiles_read(tiles_dev_ptr, ntiles, stream))


def cut_tiles(offsets: np.ndarray, src_base: int, dst_base: int) -> np.ndarray:
    """tbr_tile records (n, 3) uint64 -- src, dst, bytes | 0 << 32 -- for a
    batch of (src_off, dst_off, bytes) copies cut into tiles of at most 4 KiB,
    in the batch's order.  Every copy must be a multiple of 16 bytes with
    16-byte aligned ends (the instruments' tiles are 16-byte streams)."""
    o = np.ascontiguousarray(offsets, dtype=np.uint64).reshape(-1, 3)
    nbytes = o[:, 2].astype(np.int64)
    if np.any(nbytes % 16) or np.any(o[:, 0] % np.uint64(16)) or np.any(o[:, 1] % np.uint64(16)) \
            or (src_base | dst_base) % 16:
        raise ValueError("tiles need 16-byte aligned copies of multiples of 16 bytes")
    per = np.maximum((nbytes + TILE_BYTES - 1) // TILE_BYTES, 0)
    owner = np.repeat(np.arange(len(o)), per)
    first = np.repeat(np.cumsum(per) - per, per)
    k = np.arange(per.sum()) - first                      # tile index within its copy
    off = (k * TILE_BYTES).astype(np.uint64)
    left = nbytes[owner] - k * TILE_BYTES
    tiles = np.empty((len(owner), 3), dtype=np.uint64)
    tiles[:, 0] = o[owner, 0] + np.uint64(src_base) + off
    tiles[:, 1] = o[owner, 1] + np.uint64(dst_base) + off
    tiles[:, 2] = np.minimum(left, TILE_BYTES).astype(np.uint64)
    return tiles
