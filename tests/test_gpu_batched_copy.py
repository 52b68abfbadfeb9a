"""GPU parity of the batched copy (tb_batched_copy through the C ABI) against
the oracle's per-descriptor memcpy: every byte of the destination pool
compared, never-written bytes must keep the pool's pre-fill."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

KiB, MiB = 1024, 1 << 20


def _run_batch(torch, batch: wl.Batch, src_shift: int = 0, dst_shift: int = 0, stream=None, launches: int = 1):
    """Upload payload and pool, launch, compare the whole pool with the oracle.
    src_shift / dst_shift move the base addresses off 256-byte alignment."""
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import make_desc
    src = torch.empty(batch.src_bytes + 64, dtype=torch.uint8, device="cuda")
    if batch.src_bytes:
        src[src_shift:src_shift + batch.src_bytes].copy_(torch.from_numpy(batch.payload[:batch.src_bytes]))
    pool = torch.full((batch.pool_bytes + 64,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    desc = make_desc(batch.desc, int(src.data_ptr()) + src_shift, int(pool.data_ptr()) + dst_shift)
    s = stream or torch.cuda.current_stream()
    torch.cuda.synchronize()
    for _ in range(launches):
        tb.tb_batched_copy(int(desc.data_ptr()), batch.ncopies, s.cuda_stream)
    s.synchronize()
    got = pool.cpu().numpy()
    exp = np.full(batch.pool_bytes + 64, wl.POOL_FILL, dtype=np.uint8)
    image = np.zeros(batch.src_bytes + 64, dtype=np.uint8)
    image[src_shift:src_shift + batch.src_bytes] = batch.payload[:batch.src_bytes]
    d = batch.desc.copy()
    d[:, 0] += np.uint64(src_shift)
    d[:, 1] += np.uint64(dst_shift)
    oracle.ref_batch(exp, image, d)
    return oracle.first_mismatch(got, exp)


@pytest.mark.parametrize("seed", range(40))
def test_small_random_batches_all_alignments(seed):
    """1-64 descriptors of 0-300 bytes at arbitrary byte alignments."""
    torch = require_gpu()
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 65))
    b = wl.batch_random(seed, n, max_bytes=300, pool_bytes=1 << 16)
    note(f"batched random seed={seed} n={n} max=300")
    assert _run_batch(torch, b, src_shift=seed % 16, dst_shift=(seed * 7) % 16) == -1


@pytest.mark.parametrize("align", [1, 2, 4, 8, 16, 64])
def test_mixed_sizes_by_alignment(align):
    torch = require_gpu()
    b = wl.batch_random(77 + align, 500, max_bytes=20000, pool_bytes=16 << 20,
                        src_align=align, dst_align=align, size_align=align)
    note(f"batched 500 copies <=20000 B align={align}")
    assert _run_batch(torch, b) == -1


def test_mooncake_lengths_1B_to_3MiB_unaligned():
    """Lengths from 1 byte to 3 MiB, unaligned ranges (Design of #5040, Correctness)."""
    torch = require_gpu()
    rng = np.random.default_rng(42)
    sizes = np.unique(np.concatenate([
        [1, 2, 3, 15, 16, 17, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 4097, 65535, 65536, 65537,
         64 * KiB + 1, 100000, 1 << 20, (1 << 20) + 3, 3 * MiB - 1, 3 * MiB],
        rng.integers(1, 3 * MiB, size=20)])).astype(np.int64)
    n = len(sizes)
    src_off = np.zeros(n, np.int64)
    dst_off = np.zeros(n, np.int64)
    ps, pd = 3, 5
    for i, s in enumerate(sizes):
        src_off[i], dst_off[i] = ps, pd
        ps += int(s) + int(rng.integers(1, 40))
        pd += int(s) + int(rng.integers(1, 40))
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    perm = rng.permutation(n)
    batch = wl.Batch("mooncake_lengths", desc[perm], ps + 64, pd + 64, 42,
                     payload=wl.random_payload(rng, ps + 64))
    note(f"batched lengths 1B-3MiB n={n} unaligned")
    assert _run_batch(torch, batch) == -1


def test_large_copies_split_and_queue_reset_across_launches():
    """Copies above the split size are shared by many waves; repeated launches
    on one stream must find the queue cleared by the previous launch."""
    torch = require_gpu()
    rng = np.random.default_rng(8)
    sizes = np.array([64 * KiB + 16, 100 * KiB, 1 * MiB, 2 * MiB + 48, 8 * MiB] + [512] * 300, np.int64)
    rng.shuffle(sizes)
    n = len(sizes)
    src_off = np.concatenate([[0], np.cumsum(sizes[:-1])]).astype(np.int64)
    dst_off = (np.arange(n, dtype=np.int64) * (9 * MiB))
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    total = int(sizes.sum())
    batch = wl.Batch("split", desc, total, n * 9 * MiB, 8, payload=wl.random_payload(rng, total))
    for rep in range(3):
        note(f"batched large split rep={rep}")
        assert _run_batch(torch, batch, launches=2 + rep) == -1


def test_queue_overflow_runs_on_owner_waves():
    """More long copies than the queue holds: the overflow ones are copied by
    the wave that owns them."""
    torch = require_gpu()
    rng = np.random.default_rng(9)
    n = 16384 + 300
    size = 64 * KiB + 64
    sizes = np.full(n, size, np.int64)
    src_off = np.arange(n, dtype=np.int64) * size
    dst_off = rng.permutation(n).astype(np.int64) * (size + 64)
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    batch = wl.Batch("overflow", desc, n * size, n * (size + 64), 9, payload=wl.random_payload(rng, n * size))
    note(f"batched queue overflow n={n} size={size}")
    assert _run_batch(torch, batch, launches=2) == -1


def test_zero_length_and_empty_batches():
    import copy_reduce_amd as tb
    torch = require_gpu()
    b = wl.batch_random(5, 64, max_bytes=100, pool_bytes=1 << 14)
    b.desc[::3, 2] = 0
    note("batched with zero-length descriptors")
    assert _run_batch(torch, b) == -1
    note("batched empty batch")
    tb.tb_batched_copy(0, 0, torch.cuda.current_stream().cuda_stream)      # no-op, no device access
    torch.cuda.synchronize()


def test_two_streams_use_separate_scratch():
    torch = require_gpu()
    rng = np.random.default_rng(12)
    sizes = np.array([3 * MiB] * 6 + [4096] * 50, np.int64)
    n = len(sizes)
    src_off = np.concatenate([[0], np.cumsum(sizes[:-1])]).astype(np.int64)
    dst_off = np.arange(n, dtype=np.int64) * (4 * MiB)
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    total = int(sizes.sum())
    batch = wl.Batch("two-streams", desc, total, n * 4 * MiB, 12, payload=wl.random_payload(rng, total))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    note("batched on stream 1")
    assert _run_batch(torch, batch, stream=s1) == -1
    note("batched on stream 2")
    assert _run_batch(torch, batch, stream=s2) == -1
