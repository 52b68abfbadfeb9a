"""copy_reduce_amd: the MI355X (gfx950) transfer hot path behind a C ABI.

    libtb.so (include/tb.h)      hand-written HIP kernels + host checks
    copy_reduce_amd._tb          ctypes binding, same names as the C calls
    copy_reduce_amd.torch_api    torch-tensor conveniences (device memory and
                                 streams only; every step runs in libtb)

Importing this package loads libtb.so and fails if it has not been built:
there is no CPU or library fallback.
"""
from ._tb import (  # noqa: F401
    EXPORTS, LIB_PATH, TB_BC_NO_PIECES, TB_BC_NO_WAIT, TB_BC_NORMAL, TB_ERR_HIP, TB_ERR_INVALID, TB_ERR_NOMEM, TB_ERR_TIMEOUT, TB_MAX_SRCS, TB_OK,
    TB_RING_DIRECT, TB_RING_STAGED,
    TBError, lib, tb_batched_copy, tb_batched_copy_noalloc, tb_batched_set_mode, tb_launch_info, tb_num_slices, tb_prep_reference, tb_prep_sources,
    tb_reduce_copy, tb_ring_create, tb_ring_destroy, tb_ring_poll, tb_ring_submit, tb_ring_wait, tb_rotate_sources,
    tb_shutdown, tb_slice_stride, tb_spin_gate_arm, tb_spin_gate_release, tb_spin_gate_status, tb_status_string,
    tb_time_next_launch, tb_batched_set_max_workgroups,
)
