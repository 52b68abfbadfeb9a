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
    batch.check()
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
    rep = oracle.mismatch_report(got, exp)
    if rep is None:
        return -1
    note(f"  first differing byte {rep[0]}: expected {int(rep[1]):#04x}, got {int(rep[2]):#04x}")
    _describe_mismatch(got, exp, d)
    return rep[0]


def _describe_mismatch(got, exp, desc):
    """Print which copies differ and how (not written at all, or partly)."""
    bad = []
    for k, (s, dd, b) in enumerate(desc.astype(np.int64)):
        if b and not np.array_equal(got[dd:dd + b], exp[dd:dd + b]):
            wrong = np.flatnonzero(got[dd:dd + b] != exp[dd:dd + b])
            bad.append((k, int(s), int(dd), int(b), len(wrong), int(wrong[0]), int(wrong[-1]),
                        bool(np.all(got[dd:dd + b][wrong] == wl.POOL_FILL))))
    note(f"  {len(bad)} copies differ (index, src, dst, bytes, n_wrong, first, last, all_unwritten):")
    for row in bad[:12]:
        note(f"    {row}")


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


@pytest.mark.parametrize("mode", ["TB_BC_NORMAL", "TB_BC_NO_PIECES"])
def test_long_copies_every_relative_offset(mode):
    """Copies above the split size at every (source, destination) offset modulo
    16: pieces that start inside 16-byte blocks, realigned in registers, and
    (TB_BC_NO_PIECES) the recovery path's whole-copy routine."""
    import copy_reduce_amd as tb
    torch = require_gpu()
    rng = np.random.default_rng(16)
    size = 200 * KiB + 7
    slot = 256 * KiB
    rows = []
    ps = 0
    for so in range(16):
        for do in range(16):
            k = len(rows)
            rows.append((ps + so, k * slot + do, size))
            ps += size + 64
    desc = np.array(rows, dtype=np.uint64)
    batch = wl.Batch("long_every_offset", desc, ps + 64, len(rows) * slot, 16, payload=wl.random_payload(rng, ps + 64))
    tb.tb_batched_set_mode(getattr(tb, mode))
    try:
        note(f"batched long copies at all 256 offset pairs, mode {mode}")
        assert _run_batch(torch, batch) == -1
    finally:
        tb.tb_batched_set_mode(tb.TB_BC_NORMAL)


def test_queue_overflow_runs_on_owner_waves():
    """More long copies than the queue holds: the overflow ones are copied by
    the scanning wave that found them."""
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


def _long_and_short_batch(seed: int) -> wl.Batch:
    """300 long copies (64 KiB + 16 B to 1 MiB, some unaligned) among 1,700
    short ones, shuffled."""
    rng = np.random.default_rng(seed)
    long_sizes = rng.integers(64 * KiB + 1, 1 * MiB, size=300)
    short_sizes = rng.integers(1, 8 * KiB, size=1700)
    sizes = np.concatenate([long_sizes, short_sizes]).astype(np.int64)
    rng.shuffle(sizes)
    n = len(sizes)
    gaps_s = rng.integers(0, 48, size=n)
    gaps_d = rng.integers(0, 48, size=n)
    src_off = np.concatenate([[0], np.cumsum(sizes[:-1] + gaps_s[:-1])]).astype(np.int64)
    dst_off = np.concatenate([[0], np.cumsum(sizes[:-1] + gaps_d[:-1])]).astype(np.int64)
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    src_total = int(src_off[-1] + sizes[-1])
    pool = int(dst_off[-1] + sizes[-1]) + 64
    return wl.Batch(f"long_short_{seed}", desc, src_total, pool, seed, payload=wl.random_payload(rng, src_total))


def test_same_batch_moved_by_three_bytes_between_calls():
    """The same descriptor indices at new addresses: a launch must read the
    descriptors of its own call, never ones left from the previous call."""
    torch = require_gpu()
    batch = _long_and_short_batch(12)
    note("batched long/short shift 3 then 0")
    assert _run_batch(torch, batch, src_shift=3, dst_shift=3, launches=2) == -1
    assert _run_batch(torch, batch, launches=1) == -1


@pytest.mark.parametrize("mode", ["TB_BC_NO_WAIT", "TB_BC_NO_PIECES"])
@pytest.mark.parametrize("case", ["long_short", "c5_256MiB_pool", "overflow"])
def test_recovery_path_gives_identical_bytes(mode, case):
    """Waves that do not wait for the long-copy queue leave it to the last
    workgroup, which copies every queued copy: the bytes are the oracle's all
    the same, and a normal launch afterwards finds the scratch cleared."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    if case == "long_short":
        batch = _long_and_short_batch(12)
    elif case == "c5_256MiB_pool":
        batch = wl.batch_c5(pool_bytes=256 * MiB)
    else:
        rng = np.random.default_rng(13)
        n, size = 16384 + 40, 64 * KiB + 16
        sizes = np.full(n, size, np.int64)
        src_off = np.arange(n, dtype=np.int64) * size
        dst_off = rng.permutation(n).astype(np.int64) * (size + 64)
        desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
        batch = wl.Batch("overflow", desc, n * size, n * (size + 64), 13, payload=wl.random_payload(rng, n * size))
    note(f"batched recovery mode={mode} case={case} n={batch.ncopies}")
    tb.tb_batched_set_mode(getattr(tb, mode))
    try:
        assert _run_batch(torch, batch, src_shift=3, dst_shift=3, launches=2) == -1
        assert _run_batch(torch, batch, launches=1) == -1
    finally:
        tb.tb_batched_set_mode(tb.TB_BC_NORMAL)
    note(f"batched recovery mode={mode} case={case}: normal launch after")
    assert _run_batch(torch, batch, launches=1) == -1


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


def test_torch_conveniences_reject_out_of_range_counts():
    """The torch wrappers refuse counts beyond the tensors they were given, so
    no launch can read or write past them."""
    torch = require_gpu()
    from copy_reduce_amd.torch_api import batched_copy, reduce_copy
    desc = torch.zeros((4, 3), dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        batched_copy(desc, ncopies=5)
    with pytest.raises(ValueError):
        batched_copy(desc.view(-1))
    dst = torch.zeros(100, dtype=torch.float32, device="cuda")
    src = torch.zeros(200, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        reduce_copy(dst, [src], nfloats=101)
    with pytest.raises(ValueError):
        reduce_copy(dst, [src[:50]])
    reduce_copy(dst, [src], nfloats=100)
    batched_copy(desc, ncopies=0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["TB_BC_NORMAL", "TB_BC_NO_WAIT"])
def test_consecutive_launches_alternate_batches(mode):
    """Launches on one stream reuse one scratch: the scan words alternate by
    launch and queue slots carry the launch's number, so batches with and
    without long copies may follow each other in any order."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    batches = [_long_and_short_batch(31), wl.batch_random(32, 900, max_bytes=3000, pool_bytes=8 << 20),
               _long_and_short_batch(33)]
    order = [0, 1, 2, 0, 2, 1, 1, 0]
    tb.tb_batched_set_mode(getattr(tb, mode))
    try:
        for step, k in enumerate(order):
            note(f"batched alternating mode={mode} step={step} batch={k}")
            assert _run_batch(torch, batches[k], src_shift=step % 5, dst_shift=(3 * step) % 7) == -1
    finally:
        tb.tb_batched_set_mode(tb.TB_BC_NORMAL)


def test_shutdown_frees_scratch_and_later_calls_start_afresh():
    """tb_shutdown waits for the device and frees the library's scratch and
    gate memory; later calls allocate them again (launch numbering restarts
    on the new scratch), and a second shutdown is harmless."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    batch = _long_and_short_batch(41)
    note("batched shutdown / relaunch")
    assert _run_batch(torch, batch, launches=3) == -1
    tb.tb_shutdown()
    tb.tb_shutdown()
    assert _run_batch(torch, batch, launches=2) == -1
    stream = torch.cuda.current_stream().cuda_stream
    tb.tb_spin_gate_arm(1000, stream)
    tb.tb_spin_gate_release()
    torch.cuda.synchronize()
    assert tb.tb_spin_gate_status() == tb.TB_OK


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_refused_under_graph_capture():
    """A launch numbers itself on its scratch when enqueued, so a replayed
    capture would repeat the number: the call is refused on a capturing stream
    and enqueues nothing; the same calls work once the capture is over."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import DescRing, make_desc
    b = wl.batch_random(5, 20, max_bytes=2000, pool_bytes=1 << 20)
    src = torch.from_numpy(b.payload).cuda()
    pool = torch.full((b.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    desc = make_desc(b.desc, int(src.data_ptr()), int(pool.data_ptr()))
    host = b.desc.astype(np.uint64).copy()
    host[:, 0] += np.uint64(int(src.data_ptr()))
    host[:, 1] += np.uint64(int(pool.data_ptr()))
    torch.cuda.synchronize()
    note("batched copy refused under graph capture")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with DescRing(nslots=2, slot_descs=8, stream=side) as ring:
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                with pytest.raises(tb.TBError) as e1:
                    tb.tb_batched_copy(int(desc.data_ptr()), b.ncopies, side.cuda_stream)
                with pytest.raises(tb.TBError) as e2:
                    ring.submit(host)
        assert e1.value.status == tb.TB_ERR_INVALID and e2.value.status == tb.TB_ERR_INVALID
        torch.cuda.synchronize()
        assert bool((pool == wl.POOL_FILL).all())            # nothing ran
        # the same calls work once the capture is over
        tb.tb_batched_copy(int(desc.data_ptr()), b.ncopies, side.cuda_stream)
        side.synchronize()
    got = pool.cpu().numpy()
    exp = np.full(b.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    oracle.ref_batch(exp, b.payload, b.desc)
    oracle.assert_equal(got, exp)


def test_threads_on_their_own_streams():
    """Four host threads, each on its own stream with its own batch and pool,
    call tb_batched_copy concurrently (the library's scratch map is shared and
    locked; each stream gets its own scratch)."""
    import threading
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import make_desc
    jobs = []
    for t in range(4):
        b = wl.batch_c5(seed=40 + t, pool_bytes=64 << 20, n_block=400, n_index=100, n_mla=1)
        src = torch.from_numpy(b.payload).cuda()
        pool = torch.full((b.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
        desc = make_desc(b.desc, int(src.data_ptr()), int(pool.data_ptr()))
        jobs.append((b, src, pool, desc, torch.cuda.Stream()))
    torch.cuda.synchronize()
    note("batched copy from 4 threads on 4 streams")
    errors = []

    def work(job):
        b, _, _, desc, s = job
        try:
            for _ in range(5):
                tb.tb_batched_copy(int(desc.data_ptr()), b.ncopies, s.cuda_stream)
            s.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for b, _, pool, _, _ in jobs:
        exp = np.full(b.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
        oracle.ref_batch(exp, b.payload, b.desc)
        oracle.assert_equal(pool.cpu().numpy(), exp)


@pytest.mark.parametrize("cap", [8, 64, 1000])
def test_workgroup_cap_gives_identical_bytes(cap):
    """tb_batched_set_max_workgroups: the same bytes with the grid capped at
    8, 64 and 1,000 workgroups (each wave then owns many descriptors, and with
    8 every workgroup is also a scanner), through tb_batched_copy and a ring."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_c5(seed=60 + cap, pool_bytes=128 << 20, n_block=2500, n_index=800, n_mla=2)
    note(f"batched copy, grid capped at {cap} workgroups")
    tb.tb_batched_set_max_workgroups(cap)
    try:
        assert tb.tb_launch_info(0, 1, b.ncopies)["batched_blocks"] <= max(8, cap)
        assert _run_batch(torch, b, launches=2) == -1
        src = torch.from_numpy(b.payload).cuda()
        pool = torch.full((b.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
        host = b.desc.astype(np.uint64).copy()
        host[:, 0] += np.uint64(int(src.data_ptr()))
        host[:, 1] += np.uint64(int(pool.data_ptr()))
        torch.cuda.synchronize()
        with DescRing(nslots=4, slot_descs=1024) as ring:
            t = 0
            for a in range(0, b.ncopies, 1000):
                t = ring.submit(host[a:a + 1000])
            ring.wait(t)
    finally:
        tb.tb_batched_set_max_workgroups(0)
    exp = np.full(b.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    oracle.ref_batch(exp, b.payload, b.desc)
    oracle.assert_equal(pool.cpu().numpy(), exp)


def test_threads_sharing_one_stream():
    """Four host threads call tb_batched_copy on the same (default) stream at
    once: each launch is numbered on the stream's scratch and enqueued under
    one lock, so the launches reach the stream in the order of their numbers."""
    import threading
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import make_desc
    jobs = []
    for t in range(4):
        b = wl.batch_c5(seed=80 + t, pool_bytes=64 << 20, n_block=300, n_index=100, n_mla=1)
        src = torch.from_numpy(b.payload).cuda()
        pool = torch.full((b.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
        desc = make_desc(b.desc, int(src.data_ptr()), int(pool.data_ptr()))
        jobs.append((b, src, pool, desc))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    note("batched copy from 4 threads on one stream")
    errors = []
    start = threading.Barrier(4)

    def work(job):
        b, _, _, desc = job
        try:
            start.wait()
            for _ in range(25):
                tb.tb_batched_copy(int(desc.data_ptr()), b.ncopies, stream.cuda_stream)
        except Exception as e:  # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for b, _, pool, _ in jobs:
        exp = np.full(b.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
        oracle.ref_batch(exp, b.payload, b.desc)
        oracle.assert_equal(pool.cpu().numpy(), exp)


def _random_mixed_batch(seed):
    """A seeded batch mixing empty, tiny, unaligned, page-sized and long copies
    (some longer than the split size), destinations disjoint with random gaps."""
    rng = np.random.default_rng(9000 + seed)
    n = int(rng.choice([1, 2, 63, 64, 65, 500, 1023, 1024, 1025, 3000, 9000]))
    kind = rng.integers(0, 6, size=n)
    sizes = np.where(kind == 0, 0,
             np.where(kind == 1, rng.integers(1, 64, size=n),
             np.where(kind == 2, rng.integers(64, 4096, size=n),
             np.where(kind == 3, 64 * rng.integers(1, 257, size=n),
             np.where(kind == 4, rng.integers(60 * KiB, 70 * KiB, size=n),
                      rng.integers(64 * KiB, 2 * MiB, size=n)))))).astype(np.int64)
    if n > 100:                      # keep the total modest: long copies only in a few places
        longs = np.flatnonzero(sizes > 64 * KiB)
        sizes[longs[8:]] = rng.integers(1, 2048, size=max(0, longs.size - 8))
    align = int(rng.choice([1, 4, 16]))
    src_off, dst_off = np.zeros(n, np.int64), np.zeros(n, np.int64)
    ps = int(rng.integers(0, 16))
    for i in range(n):
        ps = (ps + align - 1) // align * align
        src_off[i] = ps
        ps += int(sizes[i]) + int(rng.integers(0, 32))
    order = rng.permutation(n)
    pd = int(rng.integers(0, 16))
    for i in order:
        pd = (pd + align - 1) // align * align
        dst_off[i] = pd
        pd += int(sizes[i]) + int(rng.integers(0, 32))
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    return wl.Batch(f"mixed{seed}", desc, ps + 64, pd + 64, seed, payload=wl.random_payload(rng, ps + 64))


@pytest.mark.parametrize("seed", range(24))
def test_seeded_mixed_batches_under_random_settings(seed):
    """24 seeded batches of every kind of copy, each under a seeded choice of
    recovery mode and workgroup cap, launched twice in a row on one stream."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    rng = np.random.default_rng(seed)
    b = _random_mixed_batch(seed)
    mode = [tb.TB_BC_NORMAL, tb.TB_BC_NORMAL, tb.TB_BC_NO_WAIT, tb.TB_BC_NO_PIECES][seed % 4]
    cap = int(rng.choice([0, 0, 8, 64, 512]))
    note(f"batched mixed seed={seed} n={b.ncopies} bytes={b.total_bytes} mode={mode} cap={cap}")
    tb.tb_batched_set_mode(mode)
    tb.tb_batched_set_max_workgroups(cap)
    try:
        assert _run_batch(torch, b, src_shift=seed % 7, dst_shift=(seed * 5) % 9, launches=2) == -1
    finally:
        tb.tb_batched_set_mode(tb.TB_BC_NORMAL)
        tb.tb_batched_set_max_workgroups(0)
