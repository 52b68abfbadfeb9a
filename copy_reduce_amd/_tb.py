"""ctypes binding of libtb.so (include/tb.h): argument marshalling only.

Every function below has the name of the C entry point it calls and raises
TBError when that call returns an error status.  All GPU work happens in the
library's kernels; nothing here computes any part of the method.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtb.so")

TB_OK = 0
TB_ERR_INVALID = -1
TB_ERR_HIP = -2
TB_ERR_NOMEM = -3
TB_ERR_TIMEOUT = -4
TB_MAX_SRCS = 16
TB_FILL_DEFAULT, TB_FILL_PATTERN, TB_FILL_COMPRESS = 0, 1, 2
TB_BC_NORMAL, TB_BC_NO_WAIT, TB_BC_NO_PIECES = 0, 1, 2
TB_RING_STAGED, TB_RING_DIRECT = 0, 1

# Every symbol include/tb.h declares.
EXPORTS = (
    "tb_num_slices", "tb_slice_stride", "tb_prep_reference", "tb_rotate_sources",
    "tb_status_string", "tb_last_hip_error", "tb_prep_sources", "tb_reduce_copy",
    "tb_reduce_copy_ex", "tb_batched_copy", "tb_batched_set_mode", "tb_spin_gate_arm", "tb_spin_gate_release",
    "tb_spin_gate_status", "tb_launch_info", "tb_shutdown",
    "tb_ring_create", "tb_ring_submit", "tb_ring_poll", "tb_ring_wait", "tb_ring_destroy",
    "tb_time_next_launch", "tb_batched_set_max_workgroups", "tb_batched_copy_noalloc",
)

# torch ships its own HIP runtime under the same soname (libamdhip64.so.7) as
# /opt/rocm's.  Loading torch first makes libtb bind to that one runtime;
# loading libtb first would bring up a second runtime that sees no device
# once torch starts its own.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()'); there is no fallback path")

lib = ctypes.CDLL(LIB_PATH)

_u64, _i64, _u32, _i32, _vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p


class tb_fill_cfg(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("compress_pct", ctypes.c_uint32 * 5),
                ("pattern", ctypes.c_void_p), ("pattern_len", ctypes.c_uint64),
                ("seed", ctypes.c_uint64)]


class tb_copy_desc(ctypes.Structure):
    _fields_ = [("src", ctypes.c_uint64), ("dst", ctypes.c_uint64), ("bytes", ctypes.c_uint64)]


_SIGS = {
    "tb_num_slices": (ctypes.c_int, [_u64, _u64, ctypes.POINTER(_u64)]),
    "tb_slice_stride": (ctypes.c_int, [_u64, ctypes.POINTER(_u64)]),
    "tb_prep_reference": (ctypes.c_int, [_vp, _u64, _i32, ctypes.POINTER(tb_fill_cfg)]),
    "tb_rotate_sources": (ctypes.c_int, [_vp, _i32, _u64, _u64, _i64, _vp]),
    "tb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tb_last_hip_error": (ctypes.c_char_p, []),
    "tb_prep_sources": (ctypes.c_int, [_vp, _u64, _u64, _vp, _u64, _vp]),
    "tb_reduce_copy": (ctypes.c_int, [_vp, _vp, _i32, _u64, _vp]),
    "tb_reduce_copy_ex": (ctypes.c_int, [_vp, _vp, _i32, _u64, _u32, _vp]),
    "tb_batched_copy": (ctypes.c_int, [_vp, _u32, _vp]),
    "tb_batched_copy_noalloc": (ctypes.c_int, [_vp, _u32, _vp]),
    "tb_batched_set_mode": (ctypes.c_int, [_i32]),
    "tb_spin_gate_arm": (ctypes.c_int, [_u32, _vp]),
    "tb_spin_gate_release": (ctypes.c_int, []),
    "tb_spin_gate_status": (ctypes.c_int, []),
    "tb_launch_info": (ctypes.c_int, [_u64, _i32, _u32, ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                      ctypes.POINTER(_i32)]),
    "tb_shutdown": (ctypes.c_int, []),
    "tb_ring_create": (ctypes.c_int, [_u32, _u32, _u32, _vp, ctypes.POINTER(_vp)]),
    "tb_ring_submit": (ctypes.c_int, [_vp, _vp, _u64, ctypes.POINTER(_u64)]),
    "tb_ring_poll": (ctypes.c_int, [_vp, _u64, ctypes.POINTER(_i32)]),
    "tb_ring_wait": (ctypes.c_int, [_vp, _u64]),
    "tb_ring_destroy": (ctypes.c_int, [_vp]),
    "tb_time_next_launch": (ctypes.c_int, [_vp, _vp]),
    "tb_batched_set_max_workgroups": (ctypes.c_int, [_u32]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class TBError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib.tb_status_string(status).decode()
        if status == TB_ERR_HIP:
            msg += ": " + lib.tb_last_hip_error().decode()
        super().__init__(f"{fn} failed with {status} ({msg})")


def _check(fn, status):
    if status != TB_OK:
        raise TBError(fn, status)


def _ptr_array(ptrs):
    n = len(ptrs)
    return (ctypes.c_void_p * max(1, n))(*[int(p) for p in ptrs])


# ---------------------------------------------------------------- host-only

def tb_num_slices(num_bytes: int, rotate_bytes: int) -> int:
    k = _u64()
    _check("tb_num_slices", lib.tb_num_slices(num_bytes, rotate_bytes, ctypes.byref(k)))
    return k.value


def tb_slice_stride(num_bytes: int) -> int:
    s = _u64()
    _check("tb_slice_stride", lib.tb_slice_stride(num_bytes, ctypes.byref(s)))
    return s.value


def make_fill_cfg(fill):
    """fill: None (default PrepSrcValue), ("pattern", floats) or ("compress", pct5, seed)."""
    cfg = tb_fill_cfg()
    keep = None
    if fill is None:
        cfg.kind = TB_FILL_DEFAULT
    elif fill[0] == "pattern":
        import numpy as np
        keep = np.ascontiguousarray(fill[1], dtype=np.float32)
        cfg.kind = TB_FILL_PATTERN
        cfg.pattern = keep.ctypes.data if keep.size else None
        cfg.pattern_len = keep.size
    elif fill[0] == "compress":
        cfg.kind = TB_FILL_COMPRESS
        for i, p in enumerate(fill[1]):
            cfg.compress_pct[i] = int(p)
        cfg.seed = int(fill[2]) & (2**64 - 1)
    else:
        raise ValueError(f"unknown fill {fill[0]!r}")
    return cfg, keep


def tb_prep_reference(host_out_ptr: int, nfloats: int, buffer_idx: int, fill=None) -> None:
    """PrepareReference into host memory at host_out_ptr (nfloats floats)."""
    cfg, keep = make_fill_cfg(fill)
    _check("tb_prep_reference", lib.tb_prep_reference(host_out_ptr, nfloats, buffer_idx, ctypes.byref(cfg)))
    del keep


def tb_rotate_sources(base_ptrs, slice_stride_bytes: int, k: int, iteration: int):
    """Device addresses of the slices iteration `iteration` reads."""
    n = len(base_ptrs)
    base = _ptr_array(base_ptrs)
    out = (ctypes.c_void_p * max(1, n))()
    _check("tb_rotate_sources", lib.tb_rotate_sources(base, n, slice_stride_bytes, k, iteration, out))
    return [int(out[i] or 0) for i in range(n)]


def tb_status_string(status: int) -> str:
    return lib.tb_status_string(status).decode()


def tb_launch_info(nfloats: int = 0, nsrc: int = 1, ncopies: int = 0):
    cu, rb, bb = _i32(), _i32(), _i32()
    _check("tb_launch_info", lib.tb_launch_info(nfloats, nsrc, ncopies, ctypes.byref(cu), ctypes.byref(rb),
                                                ctypes.byref(bb)))
    return {"cu_count": cu.value, "reduce_blocks": rb.value, "batched_blocks": bb.value}


# ---------------------------------------------------------------- GPU calls

def tb_prep_sources(dev_base_ptr: int, slice_stride_bytes: int, k: int, host_ref_ptr: int,
                    nfloats: int, stream: int) -> None:
    _check("tb_prep_sources", lib.tb_prep_sources(dev_base_ptr, slice_stride_bytes, k, host_ref_ptr, nfloats, stream))


def tb_reduce_copy(dst_ptr: int, src_ptrs, nfloats: int, stream: int, memset_byte: int = 0) -> None:
    srcs = _ptr_array(src_ptrs)
    if memset_byte == 0:
        st = lib.tb_reduce_copy(dst_ptr, srcs, len(src_ptrs), nfloats, stream)
    else:
        st = lib.tb_reduce_copy_ex(dst_ptr, srcs, len(src_ptrs), nfloats, memset_byte, stream)
    _check("tb_reduce_copy", st)


def tb_batched_copy(desc_dev_ptr: int, ncopies: int, stream: int) -> None:
    _check("tb_batched_copy", lib.tb_batched_copy(desc_dev_ptr, ncopies, stream))


def tb_batched_copy_noalloc(desc_dev_ptr: int, ncopies: int, stream: int) -> None:
    _check("tb_batched_copy_noalloc", lib.tb_batched_copy_noalloc(desc_dev_ptr, ncopies, stream))


def tb_batched_set_mode(mode: int) -> None:
    _check("tb_batched_set_mode", lib.tb_batched_set_mode(mode))


def tb_time_next_launch(start_event: int, stop_event: int) -> None:
    """The next launch this thread makes records these events (hipEvent_t handles, 0 for none)."""
    _check("tb_time_next_launch", lib.tb_time_next_launch(start_event or None, stop_event or None))


def tb_batched_set_max_workgroups(max_workgroups: int) -> None:
    _check("tb_batched_set_max_workgroups", lib.tb_batched_set_max_workgroups(max_workgroups))


def tb_spin_gate_arm(timeout_ms: int, stream: int) -> None:
    _check("tb_spin_gate_arm", lib.tb_spin_gate_arm(timeout_ms, stream))


def tb_spin_gate_release() -> None:
    _check("tb_spin_gate_release", lib.tb_spin_gate_release())


def tb_spin_gate_status() -> int:
    return int(lib.tb_spin_gate_status())


def tb_shutdown() -> None:
    _check("tb_shutdown", lib.tb_shutdown())


# ---------------------------------------------------------------- descriptor-slot ring

def tb_ring_create(nslots: int, slot_descs: int, flags: int, stream: int) -> int:
    """A new ring on the current device and `stream`; returns its handle."""
    out = _vp()
    _check("tb_ring_create", lib.tb_ring_create(nslots, slot_descs, flags, stream, ctypes.byref(out)))
    return int(out.value)


def tb_ring_submit(ring: int, host_desc_ptr: int, n: int) -> int:
    """Submit n host descriptors at host_desc_ptr; returns the ticket.  On a
    runtime failure the raised TBError carries `ticket`: the ring's last ticket,
    covering the launches of the request that were enqueued before it."""
    t = _u64()
    status = lib.tb_ring_submit(ring, host_desc_ptr, n, ctypes.byref(t))
    if status != TB_OK:
        err = TBError("tb_ring_submit", status)
        err.ticket = t.value if status == TB_ERR_HIP else None
        raise err
    return t.value


def tb_ring_poll(ring: int, ticket: int) -> bool:
    done = _i32()
    _check("tb_ring_poll", lib.tb_ring_poll(ring, ticket, ctypes.byref(done)))
    return bool(done.value)


def tb_ring_wait(ring: int, ticket: int) -> None:
    _check("tb_ring_wait", lib.tb_ring_wait(ring, ticket))


def tb_ring_destroy(ring: int) -> None:
    _check("tb_ring_destroy", lib.tb_ring_destroy(ring))
