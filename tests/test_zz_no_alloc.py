"""GPU test of tb_batched_copy_noalloc, the batched copy over the library's
static per-device scratch (for callers that cannot allocate): called through
the C ABI, its destination pool must equal, byte for byte, the pool that
tb_batched_copy writes from the same input, and the oracle's per-descriptor
memcpy.  Two calls in a row, the second with a smaller batch, so the second
runs on the scratch state the first left behind."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

MiB = 1 << 20


def _pools(torch, batch: wl.Batch, src_shift: int = 0, dst_shift: int = 0):
    """(pool written by tb_batched_copy, pool written by tb_batched_copy_noalloc,
    the oracle's pool) for one batch, as host arrays."""
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import make_desc
    batch.check()
    s = torch.cuda.current_stream()
    src = torch.zeros(batch.src_bytes + 64, dtype=torch.uint8, device="cuda")
    src[src_shift:src_shift + batch.src_bytes].copy_(torch.from_numpy(batch.payload[:batch.src_bytes]))
    pools = []
    for fn in (tb.tb_batched_copy, tb.tb_batched_copy_noalloc):
        pool = torch.full((batch.pool_bytes + 64,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
        desc = make_desc(batch.desc, int(src.data_ptr()) + src_shift, int(pool.data_ptr()) + dst_shift)
        torch.cuda.synchronize()
        fn(int(desc.data_ptr()), batch.ncopies, s.cuda_stream)
        s.synchronize()
        pools.append(pool.cpu().numpy())
        del pool, desc
    exp = np.full(batch.pool_bytes + 64, wl.POOL_FILL, dtype=np.uint8)
    image = np.zeros(batch.src_bytes + 64, dtype=np.uint8)
    image[src_shift:src_shift + batch.src_bytes] = batch.payload[:batch.src_bytes]
    d = batch.desc.copy()
    d[:, 0] += np.uint64(src_shift)
    d[:, 1] += np.uint64(dst_shift)
    oracle.ref_batch(exp, image, d)
    return pools[0], pools[1], exp


def _check(torch, batch, label, **kw):
    note(f"no-alloc batched copy: {label} ({batch.ncopies} copies, {batch.total_bytes} B)")
    ref, got, exp = _pools(torch, batch, **kw)
    oracle.assert_equal(ref, exp, f"{label}: tb_batched_copy differs from the oracle")
    oracle.assert_equal(got, ref, f"{label}: tb_batched_copy_noalloc against tb_batched_copy")


def test_noalloc_matches_batched_copy_twice_smaller_second():
    """A mixed batch whose 8 MiB copies go through the long-copy queue, then a
    smaller batch of short copies: each call equals tb_batched_copy's bytes."""
    torch = require_gpu()
    first = wl.batch_c5(seed=5, pool_bytes=256 * MiB, n_block=2000, n_index=800, n_mla=4)
    second = wl.batch_c4(seed=4, n=1500, pool_bytes=64 * MiB)
    assert second.ncopies < first.ncopies and second.total_bytes < first.total_bytes
    _check(torch, first, "first call, mixed batch with long copies")
    _check(torch, second, "second call, smaller batch")


def test_noalloc_unaligned_then_tiny():
    """Copies at arbitrary byte alignments (the realigning path), then a
    batch of a few bytes."""
    torch = require_gpu()
    _check(torch, wl.batch_random(91, 400, max_bytes=70000, pool_bytes=64 * MiB), "unaligned, up to 70,000 B",
           src_shift=3, dst_shift=9)
    _check(torch, wl.batch_random(92, 5, max_bytes=40, pool_bytes=1 << 16), "five copies of at most 40 B",
           src_shift=1, dst_shift=2)


@pytest.mark.parametrize("mode", ["no_wait", "no_pieces"])
def test_noalloc_recovery_modes(mode):
    """The recovery copy (its election word lives in the same static scratch)
    gives the same bytes, twice in a row."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    m = {"no_wait": tb.TB_BC_NO_WAIT, "no_pieces": tb.TB_BC_NO_PIECES}[mode]
    tb.tb_batched_set_mode(m)
    try:
        _check(torch, wl.batch_c5(seed=6, pool_bytes=128 * MiB, n_block=600, n_index=200, n_mla=2),
               f"{mode}, mixed batch")
        _check(torch, wl.batch_c5(seed=7, pool_bytes=64 * MiB, n_block=300, n_index=100, n_mla=1),
               f"{mode}, smaller mixed batch")
    finally:
        tb.tb_batched_set_mode(tb.TB_BC_NORMAL)


def test_noalloc_argument_checks():
    require_gpu()
    import copy_reduce_amd as tb
    assert tb.lib.tb_batched_copy_noalloc(None, 0, None) == tb.TB_OK
    assert tb.lib.tb_batched_copy_noalloc(None, 3, None) == tb.TB_ERR_INVALID
    assert tb.lib.tb_batched_copy_noalloc(0x1004, 3, None) == tb.TB_ERR_INVALID
