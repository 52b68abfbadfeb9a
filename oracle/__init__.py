"""CPU oracle for the transfer hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the oracle leg of bench.py (the CPU
baseline and the checks of the benchmark's GPU results) may import this
package.  It wraps oracle/liboracle.so (plain single-threaded C,
see oracle.c for the page and section each function follows) with numpy
arrays.  It never imports the HIP package and the HIP package never imports it.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
# TB_ORACLE_LIB lets the mutation test load a deliberately broken copy.
_LIB_PATH = os.environ.get("TB_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_u64 = ctypes.c_uint64
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _load():
    if not os.path.exists(_LIB_PATH):
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_num_slices.restype = _u64
    lib.orc_num_slices.argtypes = [_u64, _u64]
    lib.orc_slice_stride.restype = _u64
    lib.orc_slice_stride.argtypes = [_u64]
    lib.orc_slice_of.restype = _u64
    lib.orc_slice_of.argtypes = [_i64, _u64]
    lib.orc_gen_default.restype = None
    lib.orc_gen_default.argtypes = [_vp, _u64, ctypes.c_int]
    lib.orc_gen_pattern.restype = None
    lib.orc_gen_pattern.argtypes = [_vp, _u64, _vp, _u64]
    lib.orc_splitmix64.restype = _u64
    lib.orc_splitmix64.argtypes = [_u64, _u64]
    lib.orc_gen_compress.restype = ctypes.c_int
    lib.orc_gen_compress.argtypes = [_vp, _u64, ctypes.c_int, _vp, _u64]
    lib.orc_ref_reduce.restype = None
    lib.orc_ref_reduce.argtypes = [_vp, _vp, ctypes.c_int, _u64, ctypes.c_uint]
    lib.orc_ref_batch.restype = None
    lib.orc_ref_batch.argtypes = [_vp, _vp, _vp, _u64]
    lib.orc_first_mismatch.restype = _i64
    lib.orc_first_mismatch.argtypes = [_vp, _vp, _u64, _u64]
    lib.orc_mismatch_report.restype = ctypes.c_int
    lib.orc_mismatch_report.argtypes = [_vp, _vp, _u64, _u64, ctypes.POINTER(_i64), ctypes.POINTER(_u64),
                                        ctypes.POINTER(_u64)]
    lib.orc_time_ref_reduce.restype = ctypes.c_double
    lib.orc_time_ref_reduce.argtypes = [_vp, _vp, ctypes.c_int, _u64, ctypes.c_uint]
    lib.orc_time_ref_batch.restype = ctypes.c_double
    lib.orc_time_ref_batch.argtypes = [_vp, _vp, _vp, _u64]
    return lib


_lib = _load()


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def num_slices(num_bytes: int, rotate_bytes: int) -> int:
    return int(_lib.orc_num_slices(num_bytes, rotate_bytes))


def slice_stride(num_bytes: int) -> int:
    return int(_lib.orc_slice_stride(num_bytes))


def slice_of(iteration: int, k: int) -> int:
    return int(_lib.orc_slice_of(iteration, k))


def splitmix64(key: int, j: int) -> int:
    return int(_lib.orc_splitmix64(key & (2**64 - 1), j))


def gen_default(n: int, buffer_idx: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _lib.orc_gen_default(_ptr(out), n, buffer_idx)
    return out


def gen_pattern(n: int, pattern) -> np.ndarray:
    pat = np.ascontiguousarray(pattern, dtype=np.float32)
    if pat.size == 0:
        raise ValueError("empty pattern")
    out = np.empty(n, dtype=np.float32)
    _lib.orc_gen_pattern(_ptr(out), n, _ptr(pat), pat.size)
    return out


def gen_compress(n: int, buffer_idx: int, pct, seed: int) -> np.ndarray:
    p = np.ascontiguousarray(pct, dtype=np.uint32)
    assert p.size == 5
    out = np.empty(n, dtype=np.float32)
    rc = _lib.orc_gen_compress(_ptr(out), n, buffer_idx, _ptr(p), seed & (2**64 - 1))
    if rc != 0:
        raise ValueError("fillCompress percentages must sum to 100")
    return out


def gen_source(n: int, buffer_idx: int, fill=None) -> np.ndarray:
    """PrepareReference for one source buffer.

    fill: None (default PrepSrcValue), ("pattern", values) or
    ("compress", pct5, seed).
    """
    if fill is None:
        return gen_default(n, buffer_idx)
    if fill[0] == "pattern":
        return gen_pattern(n, fill[1])
    if fill[0] == "compress":
        return gen_compress(n, buffer_idx, fill[1], fill[2])
    raise ValueError(f"unknown fill {fill[0]!r}")


def _src_array(srcs):
    arrs = [np.ascontiguousarray(s, dtype=np.float32) for s in srcs]
    table = (ctypes.c_void_p * max(1, len(arrs)))(*[_ptr(a) for a in arrs])
    return arrs, table


def ref_reduce(srcs, n: int = None, memset_byte: int = 0) -> np.ndarray:
    """dstReference[len(srcs)] over n floats (n is required when srcs is empty)."""
    if n is None:
        n = int(srcs[0].size)
    arrs, table = _src_array(srcs)
    for a in arrs:
        assert a.size >= n
    out = np.empty(n, dtype=np.float32)
    _lib.orc_ref_reduce(_ptr(out), ctypes.cast(table, _vp), len(arrs), n, memset_byte)
    return out


def ref_batch(pool: np.ndarray, src_image: np.ndarray, desc: np.ndarray) -> None:
    """Apply the (src_off, dst_off, bytes) descriptors to pool, in place."""
    d = np.ascontiguousarray(desc, dtype=np.uint64).reshape(-1, 3)
    assert pool.dtype == np.uint8 and src_image.dtype == np.uint8
    if d.shape[0]:
        assert int((d[:, 1] + d[:, 2]).max()) <= pool.size
        assert int((d[:, 0] + d[:, 2]).max()) <= src_image.size
    _lib.orc_ref_batch(_ptr(pool), _ptr(src_image), _ptr(d), d.shape[0])


def first_mismatch(out: np.ndarray, expected: np.ndarray) -> int:
    """-1 if byte-identical, else the index of the first differing element."""
    a = np.ascontiguousarray(out)
    b = np.ascontiguousarray(expected)
    assert a.nbytes == b.nbytes and a.itemsize == b.itemsize
    return int(_lib.orc_first_mismatch(_ptr(a), _ptr(b), a.nbytes, a.itemsize))


def mismatch_report(out: np.ndarray, expected: np.ndarray):
    """None if byte-identical, else (index, expected, actual) of the first
    differing element, the values in the arrays' dtype ("TransferBench data
    validation", How validation works: a failure names the first differing
    element with its expected and actual values)."""
    a = np.ascontiguousarray(out)
    b = np.ascontiguousarray(expected)
    assert a.nbytes == b.nbytes and a.itemsize == b.itemsize and 1 <= a.itemsize <= 8
    idx, eb, ab = _i64(), _u64(), _u64()
    if not _lib.orc_mismatch_report(_ptr(a), _ptr(b), a.nbytes, a.itemsize, ctypes.byref(idx), ctypes.byref(eb),
                                    ctypes.byref(ab)):
        return None
    as_dtype = lambda bits: np.frombuffer(int(bits).to_bytes(8, "little")[:a.itemsize], dtype=a.dtype)[0]
    return int(idx.value), as_dtype(eb.value), as_dtype(ab.value)


def assert_equal(out: np.ndarray, expected: np.ndarray, what: str = "") -> None:
    """Raise AssertionError naming the first differing element, its expected
    and its actual value (with their bits), unless the arrays are identical."""
    rep = mismatch_report(out, expected)
    if rep is None:
        return
    i, e, a = rep
    bits = lambda v: "0x" + np.asarray(v).tobytes()[::-1].hex()
    raise AssertionError(f"{what + ': ' if what else ''}first difference at element {i}: "
                         f"expected {e.item()!r} ({bits(e)}), got {a.item()!r} ({bits(a)})")


def time_ref_reduce(srcs, n: int = None, memset_byte: int = 0):
    """(seconds, result) of one single-threaded ref_reduce call."""
    if n is None:
        n = int(srcs[0].size)
    arrs, table = _src_array(srcs)
    out = np.empty(n, dtype=np.float32)
    secs = _lib.orc_time_ref_reduce(_ptr(out), ctypes.cast(table, _vp), len(arrs), n, memset_byte)
    return float(secs), out


def time_ref_batch(pool: np.ndarray, src_image: np.ndarray, desc: np.ndarray) -> float:
    """Seconds for one single-threaded ref_batch call (pool updated in place)."""
    d = np.ascontiguousarray(desc, dtype=np.uint64).reshape(-1, 3)
    return float(_lib.orc_time_ref_batch(_ptr(pool), _ptr(src_image), _ptr(d), d.shape[0]))
