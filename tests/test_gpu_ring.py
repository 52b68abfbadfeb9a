"""GPU tests of the descriptor-slot ring (tb_ring_* through the C ABI): batched
copies submitted from host descriptor lists, in slots that are held until their
launch's event fires (Mooncake RFC #5041, Design of #5040, "Descriptor slots").
Every byte of the destination pool is compared with the oracle's
per-descriptor memcpy; the unit cases of the page's Correctness list (random
content, lengths 1 B - 3 MiB, unaligned ranges, more launches than slots) run
through both ring kinds."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

KiB, MiB = 1024, 1 << 20


class _Dev:
    """A batch's payload and pre-filled pool on the device, and the batch's
    descriptors as absolute addresses in a host array."""

    def __init__(self, torch, batch: wl.Batch):
        batch.check()
        self.torch, self.batch = torch, batch
        self.src = torch.empty(batch.src_bytes + 64, dtype=torch.uint8, device="cuda")
        if batch.src_bytes:
            self.src[:batch.src_bytes].copy_(torch.from_numpy(batch.payload[:batch.src_bytes]))
        self.pool = torch.full((batch.pool_bytes + 64,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
        d = batch.desc.astype(np.uint64).copy()
        d[:, 0] += np.uint64(int(self.src.data_ptr()))
        d[:, 1] += np.uint64(int(self.pool.data_ptr()))
        self.host_desc = d
        torch.cuda.synchronize()

    def check(self) -> None:
        """The pool against the oracle's, byte for byte (a failure names the
        first differing byte with its expected and actual value)."""
        b = self.batch
        exp = np.full(b.pool_bytes + 64, wl.POOL_FILL, dtype=np.uint8)
        image = np.zeros(b.src_bytes + 64, dtype=np.uint8)
        image[:b.src_bytes] = b.payload[:b.src_bytes]
        oracle.ref_batch(exp, image, b.desc)
        oracle.assert_equal(self.pool.cpu().numpy(), exp, "pool")


def _requests(n: int, rng, most: int):
    """Cut [0, n) into consecutive requests of 1..most descriptors."""
    cuts, i = [], 0
    while i < n:
        k = int(rng.integers(1, most + 1))
        cuts.append((i, min(n, i + k)))
        i += k
    return cuts


def _submit_all(ring, host_desc, cuts):
    tickets = [ring.submit(host_desc[a:b]) for a, b in cuts]
    assert all(t2 >= t1 for t1, t2 in zip(tickets, tickets[1:]))
    return tickets


@pytest.mark.parametrize("direct", [False, True], ids=["staged", "direct"])
@pytest.mark.parametrize("seed", range(4))
def test_random_requests_through_small_ring(direct, seed):
    """500 copies of 0-20000 B at arbitrary alignments, cut into requests of
    1-200 descriptors, through 4 slots of 64: requests span several slots and
    the ring wraps many times, so submit waits on the oldest launch."""
    torch = require_gpu()
    from copy_reduce_amd.torch_api import DescRing
    rng = np.random.default_rng(300 + seed)
    b = wl.batch_random(300 + seed, 500, max_bytes=20000, pool_bytes=16 << 20)
    dev = _Dev(torch, b)
    cuts = _requests(b.ncopies, rng, 200)
    note(f"ring random seed={seed} direct={direct} requests={len(cuts)} slots=4x64")
    with DescRing(nslots=4, slot_descs=64, direct=direct) as ring:
        tickets = _submit_all(ring, dev.host_desc, cuts)
        ring.wait(tickets[-1])
        assert all(ring.poll(t) for t in tickets)
    dev.check()


@pytest.mark.parametrize("direct", [False, True], ids=["staged", "direct"])
def test_lengths_1B_to_3MiB_one_request_each(direct):
    """Lengths from 1 byte to 3 MiB at unaligned addresses, one descriptor per
    request, through 2 slots: more launches than slots, long copies split."""
    torch = require_gpu()
    from copy_reduce_amd.torch_api import DescRing
    rng = np.random.default_rng(51)
    sizes = np.unique(np.concatenate([
        [1, 2, 3, 15, 16, 17, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 4097, 65535, 65536, 65537,
         100000, 1 << 20, (1 << 20) + 3, 3 * MiB - 1, 3 * MiB],
        rng.integers(1, 3 * MiB, size=12)])).astype(np.int64)
    n = len(sizes)
    src_off, dst_off = np.zeros(n, np.int64), np.zeros(n, np.int64)
    ps, pd = 3, 5
    for i, s in enumerate(sizes):
        src_off[i], dst_off[i] = ps, pd
        ps += int(s) + int(rng.integers(1, 40))
        pd += int(s) + int(rng.integers(1, 40))
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)[rng.permutation(n)]
    b = wl.Batch("ring_lengths", desc, ps + 64, pd + 64, 51, payload=wl.random_payload(rng, ps + 64))
    dev = _Dev(torch, b)
    note(f"ring lengths 1B-3MiB direct={direct} n={n} one per request, 2 slots")
    with DescRing(nslots=2, slot_descs=8, direct=direct) as ring:
        tickets = _submit_all(ring, dev.host_desc, [(i, i + 1) for i in range(n)])
        assert tickets == list(range(1, n + 1))
        ring.wait(tickets[-1])
    dev.check()


@pytest.mark.parametrize("direct", [False, True], ids=["staged", "direct"])
def test_mixed_kv_batch_in_page_sized_requests(direct):
    """The mixed KV shape (block pages, index pages, two 8 MiB landing slots)
    in requests of at most 4,096 copies, through 32 slots of 8,192."""
    torch = require_gpu()
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_c5(seed=5, pool_bytes=256 << 20, n_block=3000, n_index=1600, n_mla=2)
    dev = _Dev(torch, b)
    cuts = [(i, min(b.ncopies, i + 4096)) for i in range(0, b.ncopies, 4096)]
    note(f"ring mixed kv direct={direct} n={b.ncopies} requests={len(cuts)}")
    with DescRing(direct=direct) as ring:
        tickets = _submit_all(ring, dev.host_desc, cuts)
        ring.wait(tickets[-1])
    dev.check()


def test_tickets_poll_wait_and_empty_submits():
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_random(11, 40, max_bytes=5000, pool_bytes=1 << 20)
    dev = _Dev(torch, b)
    note("ring tickets / poll / wait")
    with DescRing(nslots=3, slot_descs=16) as ring:
        assert ring.submit(dev.host_desc[:0]) == 0          # nothing launched yet
        assert ring.poll(0)
        with pytest.raises(tb.TBError) as ei:
            ring.poll(1)                                     # not handed out
        assert ei.value.status == tb.TB_ERR_INVALID
        t1 = ring.submit(dev.host_desc[:16])                 # one slot
        assert t1 == 1
        t2 = ring.submit(dev.host_desc[16:40])               # 24 descriptors: two slots
        assert t2 == 3
        assert ring.submit(dev.host_desc[:0]) == 3          # empty: the last launch's ticket
        with pytest.raises(tb.TBError):
            ring.wait(4)
        ring.wait(t2)
        assert ring.poll(1) and ring.poll(2) and ring.poll(3)
    dev.check()


def test_bad_descriptor_rejects_whole_request():
    """A request whose last descriptor has a NULL source is refused before any
    part of it is enqueued: the ticket count and the pool stay as they were."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_random(12, 30, max_bytes=3000, pool_bytes=1 << 20)
    dev = _Dev(torch, b)
    note("ring bad descriptor")
    with DescRing(nslots=2, slot_descs=8) as ring:
        for field, value in ((0, 0), (1, 0), (0, 2**64 - 16), (1, 2**64 - 16)):
            bad = dev.host_desc.copy()
            bad[-1, 2] = max(int(bad[-1, 2]), 32)
            bad[-1, field] = value
            with pytest.raises(tb.TBError) as ei:
                ring.submit(bad)
            assert ei.value.status == tb.TB_ERR_INVALID
            assert ring.submit(bad[:0]) == 0
        # a zero-length descriptor may carry NULL addresses
        ok = dev.host_desc.copy()
        ok[0] = (0, 0, 0)
        t = ring.submit(ok)
        ring.wait(t)
    exp_batch = wl.Batch(b.name, np.concatenate([[[0, 0, 0]], b.desc[1:]]).astype(np.uint64), b.src_bytes,
                         b.pool_bytes, b.seed, payload=b.payload)
    dev.batch = exp_batch
    dev.check()


@pytest.mark.parametrize("direct", [False, True], ids=["staged", "direct"])
def test_destroy_waits_for_work_in_flight(direct):
    torch = require_gpu()
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_c4(seed=4, n=6000, pool_bytes=256 << 20)
    dev = _Dev(torch, b)
    note(f"ring destroy with launches in flight direct={direct}")
    ring = DescRing(nslots=8, slot_descs=1024, direct=direct)
    for a in range(0, b.ncopies, 1000):
        ring.submit(dev.host_desc[a:a + 1000])
    ring.close()                     # no wait before: destroy must wait itself
    dev.check()


@pytest.mark.parametrize("mode", ["no_wait", "no_pieces"])
def test_recovery_modes_through_ring(mode):
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_c5(seed=9, pool_bytes=128 << 20, n_block=800, n_index=300, n_mla=3)
    dev = _Dev(torch, b)
    note(f"ring recovery mode={mode}")
    tb.tb_batched_set_mode(tb.TB_BC_NO_WAIT if mode == "no_wait" else tb.TB_BC_NO_PIECES)
    try:
        with DescRing(nslots=4, slot_descs=512, direct=True) as ring:
            t = 0
            for a in range(0, b.ncopies, 500):
                t = ring.submit(dev.host_desc[a:a + 500])
            ring.wait(t)
    finally:
        tb.tb_batched_set_mode(tb.TB_BC_NORMAL)
    dev.check()


@pytest.mark.parametrize("direct", [False, True], ids=["staged", "direct"])
def test_ring_and_plain_calls_interleave_on_one_stream(direct):
    """Ring launches and tb_batched_copy launches on the same stream use
    different scratch and run in stream order."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_c5(seed=21, pool_bytes=128 << 20, n_block=1200, n_index=400, n_mla=2)
    dev = _Dev(torch, b)
    dd = torch.from_numpy(dev.host_desc.view(np.int64)).cuda()
    s = torch.cuda.current_stream()
    note(f"ring + plain batched copies interleaved direct={direct}")
    with DescRing(nslots=4, slot_descs=256, direct=direct) as ring:
        t = 0
        for k, a in enumerate(range(0, b.ncopies, 300)):
            m = min(300, b.ncopies - a)
            if k % 2:
                tb.tb_batched_copy(int(dd[a:].data_ptr()), m, s.cuda_stream)
            else:
                t = ring.submit(dev.host_desc[a:a + m])
        ring.wait(t)
        s.synchronize()
    dev.check()


def test_two_rings_from_two_threads():
    """Each host thread drives its own ring on its own stream (a ring is used
    by one thread at a time; two rings are independent)."""
    import threading
    torch = require_gpu()
    from copy_reduce_amd.torch_api import DescRing
    devs = [_Dev(torch, wl.batch_c5(seed=70 + t, pool_bytes=64 << 20, n_block=600, n_index=200, n_mla=1))
            for t in range(2)]
    streams = [torch.cuda.Stream() for _ in devs]
    note("two rings, two threads")
    errors = []

    def work(dev, s, direct):
        try:
            with DescRing(nslots=4, slot_descs=128, direct=direct, stream=s) as ring:
                t = 0
                for a in range(0, dev.batch.ncopies, 100):
                    t = ring.submit(dev.host_desc[a:a + 100])
                ring.wait(t)
        except Exception as e:  # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(d, s, k == 1)) for k, (d, s) in enumerate(zip(devs, streams))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for dev in devs:
        dev.check()


@pytest.mark.parametrize("direct", [False, True], ids=["staged", "direct"])
def test_timing_hook_on_a_ring_launch(direct):
    """tb_time_next_launch before a ring submit: the launch records the start
    event and its slot's completion event, and the hook's stop event is
    recorded after it too (it is not dropped)."""
    torch = require_gpu()
    from copy_reduce_amd.torch_api import DescRing
    b = wl.batch_c4(seed=9, n=3000, pool_bytes=64 << 20)
    dev = _Dev(torch, b)
    s = torch.cuda.current_stream()
    st, sp, ref = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    st.record(s)
    sp.record(s)
    ref.record(s)                                 # later than both first records
    torch.cuda.synchronize()
    note(f"ring timing hook direct={direct}")
    with DescRing(nslots=2, slot_descs=4096, direct=direct, stream=s) as ring:
        import copy_reduce_amd as tb
        tb.tb_time_next_launch(st.cuda_event, sp.cuda_event)
        t = ring.submit(dev.host_desc)
        ring.wait(t)
        torch.cuda.synchronize()
    assert ref.elapsed_time(st) > 0.0             # recorded again, by the launch
    assert ref.elapsed_time(sp) > ref.elapsed_time(st)
    assert 0.0 < st.elapsed_time(sp) < 50.0
    dev.check()
