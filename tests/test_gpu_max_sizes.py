"""Buffers above the reduce-copy's grid cap and above 4 GiB.  The reduce-copy
kernels cap their grid at 2^20 workgroups and loop over the tiles beyond it:
the memset's 4 KiB tiles pass the cap above 4 GiB, the vector path's 1 KiB
tiles (one or two sources) above 1 GiB per buffer and its 2 KiB tiles (three
sources and more) above 2 GiB, the unaligned path's 2 KiB tiles (up to seven
sources) above 2 GiB and its LDS-staged 1 KiB tiles (eight and more) above
1 GiB.  The oracle's
definitions hold at any size and are checked as such: every byte of a memset
is the memset byte and a one-source reduce-copy equals its source bitwise
(both on the device), and every element of a multi-source sum equals the
oracle's (TransferBench data validation, Expected destination), compared in
contiguous chunks."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import GUARD_BYTE, DevBuf, note, require_gpu

pytestmark = pytest.mark.gpu

N_BIG = (1 << 30) + 1027          # floats: 4 GiB + 4,108 bytes


def _guards_on_device(buf) -> bool:
    return bool((buf.t[:buf.start] == GUARD_BYTE).all()) and bool((buf.t[buf.start + buf.nbytes:] == GUARD_BYTE).all())


def _body(buf):
    return buf.t[buf.start:buf.start + buf.nbytes]


def _fill_pattern(torch, buf, salt: int):
    """Arbitrary 32-bit patterns (NaNs and subnormals included) made on the device."""
    i = torch.arange(buf.nbytes // 4, dtype=torch.int64, device="cuda")
    _body(buf).view(torch.int32).copy_(((i * 2654435761 + salt) & 0xFFFFFFFF).to(torch.int64).sub(1 << 31).to(torch.int32))
    del i


def test_memset_above_4GiB():
    torch = require_gpu()
    import copy_reduce_amd as tb
    note(f"max size: memset n={N_BIG} byte=0x5A dst offset 4")
    buf = DevBuf(torch, N_BIG * 4, offset=4, fill=0x11)
    tb.tb_reduce_copy(buf.ptr, [], N_BIG, torch.cuda.current_stream().cuda_stream, 0x5A)
    torch.cuda.synchronize()
    assert bool((_body(buf) == 0x5A).all())
    assert _guards_on_device(buf)


def test_copy_above_4GiB_bitwise():
    torch = require_gpu()
    import copy_reduce_amd as tb
    note(f"max size: one-source copy n={N_BIG} offsets 4/4")
    src = DevBuf(torch, N_BIG * 4, offset=4)
    _fill_pattern(torch, src, 7)
    dst = DevBuf(torch, N_BIG * 4, offset=4, fill=0x11)
    tb.tb_reduce_copy(dst.ptr, [src.ptr], N_BIG, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(_body(dst), _body(src))
    assert _guards_on_device(dst)


CHUNK = 64 << 20                  # floats per comparison chunk (256 MiB per buffer)


def _compare_all_chunks(torch, dst, srcs, n):
    """Every element of dst against the oracle's fixed-order sum, 256 MiB of
    each buffer at a time.  Chunks are read back as contiguous slices (plain
    device-to-host copies): torch's advanced-index gather faulted on buffers
    whose byte offsets pass 2^32, so no index kernel touches them."""
    fd = _body(dst).view(torch.float32)
    fs = [_body(b).view(torch.float32) for b in srcs]
    for lo in range(0, n, CHUNK):
        hi = min(lo + CHUNK, n)
        got = fd[lo:hi].cpu().numpy()
        exp = oracle.ref_reduce([f[lo:hi].cpu().numpy() for f in fs])
        oracle.assert_equal(got, exp, f"chunk at element {lo}")
        del got, exp


def _fill_finite(torch, buf, n, mul, add):
    """Finite values, so the sum is the exact binary32 definition the oracle computes."""
    i = torch.arange(n, dtype=torch.int64, device="cuda")
    _body(buf).view(torch.float32).copy_(((i * mul + add) % 65521 - 32760).to(torch.float32) * 0.001)
    del i


def test_reduce2_above_4GiB_every_element():
    torch = require_gpu()
    import copy_reduce_amd as tb
    note(f"max size: two-source sum n={N_BIG}, every element against the oracle")
    a = DevBuf(torch, N_BIG * 4)
    b = DevBuf(torch, N_BIG * 4)
    _fill_finite(torch, a, N_BIG, 40503, 1)
    _fill_finite(torch, b, N_BIG, 40503, 2)
    dst = DevBuf(torch, N_BIG * 4, fill=0x11)
    tb.tb_reduce_copy(dst.ptr, [a.ptr, b.ptr], N_BIG, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    _compare_all_chunks(torch, dst, [a, b], N_BIG)
    assert _guards_on_device(dst)


@pytest.mark.parametrize("nsrc,n,offset,src_step", [
    (5, (1 << 29) + 515, 8, 0),    # 2 GiB + 2,060 B per source: the vector path's 2 KiB tiles past the grid cap
    (3, (96 << 20) + 5, 4, 0),     # 384 MiB + 20 B per source: above the memory-side cache's size
    (2, (1 << 29) + 261, 0, 4),    # 2 GiB + 1,044 B, sources 4 / 8 B off dst: the unaligned path past the cap
    (5, (1 << 29) + 261, 0, 4),    # the same with sources 4/8/12/0/4 B off
    (9, (1 << 28) + 261, 0, 4),    # 1 GiB + 1,044 B, nine sources off dst: the LDS-staged path's 1 KiB tiles past the cap
])
def test_reduce_multi_source_large_every_element(nsrc, n, offset, src_step):
    torch = require_gpu()
    import copy_reduce_amd as tb
    note(f"max size: {nsrc}-source sum n={n} offset {offset} source step {src_step}, every element against the oracle")
    srcs = [DevBuf(torch, n * 4, offset=(offset + src_step * (k + 1)) % 16) for k in range(nsrc)]
    for k, buf in enumerate(srcs):
        _fill_finite(torch, buf, n, 40503 + 2 * k, k)
    dst = DevBuf(torch, n * 4, offset=offset, fill=0x11)
    tb.tb_reduce_copy(dst.ptr, [b.ptr for b in srcs], n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    _compare_all_chunks(torch, dst, srcs, n)
    assert _guards_on_device(dst)
    del srcs
    torch.cuda.empty_cache()


def test_batched_copy_millions_of_descriptors():
    """4,500,000 copies of 1-48 bytes at arbitrary alignments plus three long
    copies: more descriptors than the largest grid has waves times 64, so every
    wave walks several 64-descriptor blocks, and thousands of scanner
    workgroups publish.  Compared with the oracle byte for byte."""
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import make_desc
    torch = require_gpu()
    rng = np.random.default_rng(77)
    n_small, MiB = 4_500_000, 1 << 20
    sizes = rng.integers(1, 49, size=n_small).astype(np.int64)
    long_sizes = np.array([3 * MiB + 5, MiB, 200_000], np.int64)
    sizes = np.concatenate([long_sizes[:1], sizes[:n_small // 2], long_sizes[1:2], sizes[n_small // 2:], long_sizes[2:]])
    n = sizes.size
    # sources packed with 0-15 bytes of slack; destinations packed in a shuffled order with 0-7 bytes of slack
    src_off = np.cumsum(np.concatenate([[0], sizes[:-1] + rng.integers(0, 16, size=n - 1)])).astype(np.int64)
    order = rng.permutation(n)
    gaps = rng.integers(0, 8, size=n)
    dst_sorted = np.cumsum(np.concatenate([[0], (sizes[order] + gaps[order])[:-1]])).astype(np.int64)
    dst_off = np.empty(n, np.int64)
    dst_off[order] = dst_sorted
    src_bytes = int(src_off[-1] + sizes[-1])
    pool_bytes = int(dst_off.max() + sizes.max() + 64)
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    batch = wl.Batch("millions", desc, src_bytes, pool_bytes, 77, payload=wl.random_payload(rng, src_bytes))
    info = tb.tb_launch_info(0, 1, n)
    note(f"max size: batched copy of {n} descriptors, grid {info['batched_blocks']} workgroups")
    assert n > 64 * 4 * info["batched_blocks"]
    src = torch.from_numpy(batch.payload).cuda()
    pool = torch.full((pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    d = make_desc(desc, int(src.data_ptr()), int(pool.data_ptr()))
    torch.cuda.synchronize()
    tb.tb_batched_copy(int(d.data_ptr()), n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    exp = np.full(pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    oracle.ref_batch(exp, batch.payload, desc)
    oracle.assert_equal(pool.cpu().numpy(), exp)


def test_batched_copy_of_one_copy_above_4GiB():
    """One descriptor of 4 GiB + 4,109 bytes (its ends 7 bytes past 16-byte
    boundaries on both sides, so a byte head, a vector body and a byte tail)
    among 300 small copies: the long copy is cut into more than half a million
    pieces.  Compared on the device: every destination equals its source, and
    the guard bytes around the pool are untouched."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import make_desc
    big = (4 << 30) + 4109
    note(f"max size: batched copy with one {big}-byte copy and 300 small ones")
    rng = np.random.default_rng(31)
    small = rng.integers(1, 3000, size=300).astype(np.int64)
    n = 301
    sizes = np.concatenate([[big], small])
    src_off = np.zeros(n, np.int64)
    dst_off = np.zeros(n, np.int64)
    ps, pd = 7, 23                                     # both 7 mod 16
    for i in range(n):
        src_off[i], dst_off[i] = ps, pd
        ps += int(sizes[i]) + 16 + int(rng.integers(0, 16))
        pd += int(sizes[i]) + 16 + int(rng.integers(0, 16))
    perm = rng.permutation(n)
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)[perm]
    src = DevBuf(torch, ps - ps % 4, offset=0)
    _fill_pattern(torch, src, 3)
    assert src.nbytes >= int((src_off + sizes).max())
    dst = DevBuf(torch, pd, offset=0, fill=0x11)
    d = make_desc(desc, src.ptr, dst.ptr)
    torch.cuda.synchronize()
    tb.tb_batched_copy(int(d.data_ptr()), n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    sb, db = _body(src), _body(dst)
    for s_, d_, b_ in desc.astype(np.int64):
        assert torch.equal(db[d_:d_ + b_], sb[s_:s_ + b_]), (s_, d_, b_)
    # bytes between destinations keep the fill (contiguous slices only: no
    # advanced indexing on a tensor this large)
    pos = 0
    for _, d_, b_ in sorted(desc.astype(np.int64).tolist(), key=lambda r: r[1]):
        if d_ > pos:
            assert bool((db[pos:d_] == 0x11).all()), (pos, d_)
        pos = d_ + b_
    assert bool((db[pos:] == 0x11).all())
    assert _guards_on_device(dst)
