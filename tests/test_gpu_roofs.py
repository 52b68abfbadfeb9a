"""GPU tests of the measuring instruments (libtb_roofs): what they read,
write and copy is what their header says, so the roofs bench.py --roofs
reports are rates of the stated work.  The tile copy of a batch is compared
with the oracle's per-descriptor memcpy, byte for byte."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu


def test_write_streams_write_every_word():
    torch = require_gpu()
    import copy_reduce_amd.roofs as rf
    sh = torch.cuda.current_stream().cuda_stream
    for nbufs, nbytes, pol in ((1, 4096 * 33 + 48, rf.TBR_STORE_STREAMING), (3, 1 << 20, rf.TBR_STORE_DEVICE),
                               (17, 4096 * 5 + 16, rf.TBR_STORE_STREAMING)):
        note(f"roofs: write {nbufs} buffers of {nbytes} B policy {pol}")
        bufs = [torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda") for _ in range(nbufs)]
        rf.tbr_write([int(b.data_ptr()) for b in bufs], nbytes, 0x01020304, pol, sh)
        torch.cuda.synchronize()
        for b in bufs:
            w = b[:nbytes].view(torch.int32)
            assert bool((w == 0x01020304).all())
            assert bool((b[nbytes:] == 0).all())


def test_read_streams_run_and_write_nothing():
    torch = require_gpu()
    import copy_reduce_amd.roofs as rf
    sh = torch.cuda.current_stream().cuda_stream
    bufs = [torch.full((4096 * 9 + 32,), k + 1, dtype=torch.uint8, device="cuda") for k in range(5)]
    before = [b.clone() for b in bufs]
    note("roofs: read 5 buffers")
    rf.tbr_read([int(b.data_ptr()) for b in bufs], 4096 * 9 + 32, sh)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(bufs, before))


def test_copy_equals_source():
    torch = require_gpu()
    import copy_reduce_amd.roofs as rf
    sh = torch.cuda.current_stream().cuda_stream
    for pol in (rf.TBR_STORE_STREAMING, rf.TBR_STORE_DEVICE):
        nbytes = 4096 * 100 + 272
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
        dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
        note(f"roofs: copy {nbytes} B policy {pol}")
        rf.tbr_copy(int(dst.data_ptr()), int(src.data_ptr()), nbytes, pol, sh)
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes], src) and bool((dst[nbytes:] == 0).all())


def test_combine_writes_the_xor_of_its_sources():
    """tbr_combine (N streams read, their XOR written to one more): every
    16-byte word of dst is the XOR of the sources' words, computed here with
    numpy on the host, and nothing past dst's end is written."""
    torch = require_gpu()
    import copy_reduce_amd.roofs as rf
    sh = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(8)
    for nsrc, nbytes, pol in ((1, 4096 * 3 + 16, rf.TBR_STORE_NT), (2, 4096 * 33 + 48, rf.TBR_STORE_STREAMING),
                              (9, 1 << 20, rf.TBR_STORE_DEVICE), (16, 4096 * 5 + 272, rf.TBR_STORE_NT)):
        note(f"roofs: combine {nsrc} sources of {nbytes} B policy {pol}")
        host = [rng.integers(0, 256, size=nbytes, dtype=np.uint8) for _ in range(nsrc)]
        srcs = [torch.from_numpy(h).cuda() for h in host]
        dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
        rf.tbr_combine([int(x.data_ptr()) for x in srcs], int(dst.data_ptr()), nbytes, pol, sh)
        torch.cuda.synchronize()
        exp = np.bitwise_xor.reduce(np.stack(host), axis=0)
        got = dst.cpu().numpy()
        oracle.assert_equal(got[:nbytes], exp, f"combine nsrc={nsrc}")
        assert not got[nbytes:].any()


@pytest.mark.parametrize("placement", ["random_slots", "packed"])
def test_tile_copy_of_c4_equals_oracle(placement):
    """C4's copies (in a 256 MiB pool) cut into tiles and copied by the
    instrument: the pool equals the oracle's, untouched bytes keep the fill;
    then written-only tiles leave exactly the copies' bytes rewritten."""
    torch = require_gpu()
    import copy_reduce_amd.roofs as rf
    sh = torch.cuda.current_stream().cuda_stream
    base = wl.batch_c4(n=4000, pool_bytes=256 << 20) if placement == "random_slots" else None
    batch = base if base is not None else wl.batch_c4_placed("packed", pool_bytes=4 << 30)
    if base is None:   # keep the packed case small: its first 4,000 copies
        d = batch.desc[:4000]
        batch = wl.Batch("packed4000", d, int((d[:, 0] + d[:, 2]).max()), int((d[:, 1] + d[:, 2]).max()), 4,
                         payload=batch.payload[:int((d[:, 0] + d[:, 2]).max())])
    batch.check()
    src = torch.from_numpy(batch.payload).cuda()
    pool = torch.full((batch.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    t = rf.cut_tiles(batch.desc, int(src.data_ptr()), int(pool.data_ptr()))
    tiles = torch.from_numpy(t.view(np.int64)).cuda()
    note(f"roofs: tile copy of {batch.ncopies} copies ({t.shape[0]} tiles), {placement}")
    rf.tbr_tiles_copy(int(tiles.data_ptr()), t.shape[0], rf.TBR_STORE_STREAMING, sh)
    torch.cuda.synchronize()
    exp = np.full(batch.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    oracle.ref_batch(exp, batch.payload, batch.desc)
    oracle.assert_equal(pool.cpu().numpy(), exp)
    rf.tbr_tiles_read(int(tiles.data_ptr()), t.shape[0], sh)
    rf.tbr_tiles_write(int(tiles.data_ptr()), t.shape[0], 0x5A5A5A5A, rf.TBR_STORE_DEVICE, sh)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    written = np.zeros(batch.pool_bytes, dtype=bool)
    for _, d, b in batch.desc.astype(np.int64):
        written[d:d + b] = True
    assert np.all(got[written] == 0x5A) and np.all(got[~written] == wl.POOL_FILL)
