"""GPU parity of the reduce-copy (tb_reduce_copy through the C ABI) against the
oracle: bit-exact, every N from 0 to 16, ragged sizes, independent pointer
offsets, in-place alias, special values, rotation selection, source prep."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import DevBuf, note, require_gpu

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 3, 4, 5, 63, 64, 65, 1023, 1025, 4096 * 3 + 7, (1 << 20) + 7]


def _sources(nsrc, n, kind="compress", seed=3):
    if kind == "compress":
        return [oracle.gen_compress(n, b, wl.C3_PCT, seed) for b in range(nsrc)]
    return [oracle.gen_default(n, b) for b in range(nsrc)]


def _run(torch, srcs, n, dst_off=0, src_offs=None, memset_byte=0, prefill=0xFF):
    import copy_reduce_amd as tb
    nsrc = len(srcs)
    src_offs = src_offs or [0] * nsrc
    sbufs = [DevBuf(torch, n * 4, o).upload(s[:n]) for s, o in zip(srcs, src_offs)]
    dbuf = DevBuf(torch, n * 4, dst_off, fill=prefill)
    stream = torch.cuda.current_stream().cuda_stream
    tb.tb_reduce_copy(dbuf.ptr, [b.ptr for b in sbufs], n, stream, memset_byte)
    torch.cuda.synchronize()
    got = dbuf.download().view(np.float32) if n else np.zeros(0, np.float32)
    exp = oracle.ref_reduce([s[:n] for s in srcs], n=n, memset_byte=memset_byte)
    return got, exp, dbuf, sbufs


@pytest.mark.parametrize("nsrc", list(range(0, 17)))
@pytest.mark.parametrize("n", SIZES)
def test_reduce_copy_all_n_ragged(nsrc, n):
    torch = require_gpu()
    note(f"reduce_copy nsrc={nsrc} n={n} compress seed=3")
    srcs = _sources(nsrc, n)
    got, exp, dbuf, _ = _run(torch, srcs, n)
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("offs", [(d, s0, s1) for d in (0, 4, 8, 12) for s0 in (0, 4, 8, 12) for s1 in (0, 4, 8, 12)])
def test_reduce_copy_pointer_offsets_n2(offs):
    torch = require_gpu()
    n = 4096 + 13
    note(f"reduce_copy nsrc=2 n={n} offsets={offs}")
    got, exp, dbuf, _ = _run(torch, _sources(2, n), n, dst_off=offs[0], src_offs=list(offs[1:]))
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("nsrc", list(range(1, 17)))
@pytest.mark.parametrize("off", [4, 8, 12])
@pytest.mark.parametrize("n", [5, 1029, 3 * 512 + 7, 64 * 1024 + 9])
def test_reduce_copy_congruent_offsets_all_n(nsrc, off, n):
    """Every pointer at the same offset from 16-byte alignment: the vector path
    with 1-3 head floats and a ragged tail, over several tiles of each shape."""
    torch = require_gpu()
    note(f"reduce_copy nsrc={nsrc} n={n} all offsets {off}")
    got, exp, dbuf, _ = _run(torch, _sources(nsrc, n, seed=nsrc), n, dst_off=off, src_offs=[off] * nsrc)
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("nsrc", list(range(1, 17)))
@pytest.mark.parametrize("dst_off", [0, 4, 8, 12])
@pytest.mark.parametrize("n", [7, 2053, 64 * 1024 + 3])
def test_reduce_copy_mixed_offsets_all_n(nsrc, dst_off, n):
    """Source k at offset 4(k + 1) mod 16: sources that disagree with dst and
    with each other modulo 16 (the unaligned path; one source in four lines up
    with dst when dst's offset is a multiple of 4 among them)."""
    torch = require_gpu()
    offs = [(4 * (k + 1)) % 16 for k in range(nsrc)]
    note(f"reduce_copy nsrc={nsrc} n={n} dst offset {dst_off} source offsets {offs}")
    got, exp, dbuf, _ = _run(torch, _sources(nsrc, n, seed=nsrc + 100), n, dst_off=dst_off, src_offs=offs)
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("nsrc", [1, 2, 3, 4, 7, 8, 9, 12, 16])
@pytest.mark.parametrize("body_blocks", [1, 63, 64, 65, 127, 128, 129, 255, 256, 257])
@pytest.mark.parametrize("tail", [0, 3])
def test_reduce_copy_unaligned_tile_edges(nsrc, body_blocks, tail):
    """Unaligned path (sources 4, 8, 12, 0 bytes off dst) with the float4 body
    ending on, just before and just after the edges of a wave and of a tile
    (128 blocks up to seven sources; 64-block one-wave tiles staged through LDS
    from eight up), past the first 256 blocks: the last thread's 16-byte loads
    end exactly at the sources' last body elements, and the LDS path's clamp
    to the last source block is exercised at every offset."""
    torch = require_gpu()
    tile = 128
    n = 4 * (2 * tile + body_blocks) + tail
    offs = [(4 * (k + 1)) % 16 for k in range(nsrc)]
    note(f"reduce_copy unaligned nsrc={nsrc} n={n} source offsets {offs}")
    got, exp, dbuf, _ = _run(torch, _sources(nsrc, n, seed=body_blocks + tail), n, dst_off=0, src_offs=offs)
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("nsrc", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("body_blocks", [1, 63, 64, 65, 127, 128, 129])
def test_reduce_copy_vector_tile_edges(nsrc, body_blocks):
    """Vector path with the float4 body ending at and around the edges of a
    wave and of a tile (64 blocks up to two sources, 128 from three), two
    tiles in, dst and sources 4 bytes past a 16-byte boundary (a head of three
    floats) and a tail of two floats."""
    torch = require_gpu()
    tile = 64 if nsrc <= 2 else 128
    n = 3 + 4 * (2 * tile + body_blocks) + 2
    note(f"reduce_copy vector nsrc={nsrc} n={n} all offsets 4")
    got, exp, dbuf, _ = _run(torch, _sources(nsrc, n, seed=body_blocks), n, dst_off=4, src_offs=[4] * nsrc)
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("seed", range(12))
def test_reduce_copy_pointer_offsets_random(seed):
    torch = require_gpu()
    rng = np.random.default_rng(seed)
    nsrc = int(rng.integers(1, 17))
    n = int(rng.integers(1, 70000))
    offs = [int(x) * 4 for x in rng.integers(0, 4, size=nsrc + 1)]
    note(f"reduce_copy nsrc={nsrc} n={n} offsets={offs}")
    got, exp, dbuf, _ = _run(torch, _sources(nsrc, n, seed=seed), n, dst_off=offs[0], src_offs=offs[1:])
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("nsrc", [1, 2, 4])
def test_reduce_copy_default_pattern_large(nsrc):
    torch = require_gpu()
    n = (1 << 22) + 3
    note(f"reduce_copy nsrc={nsrc} n={n} default pattern")
    got, exp, _, _ = _run(torch, _sources(nsrc, n, "default"), n)
    oracle.assert_equal(got, exp)


@pytest.mark.parametrize("mb", [0x00, 0x5A, 0xFF])
def test_reduce_copy_memset_byte(mb):
    torch = require_gpu()
    n = 100003
    note(f"reduce_copy nsrc=0 n={n} memset={mb:#x}")
    got, exp, dbuf, _ = _run(torch, [], n, dst_off=4, memset_byte=mb, prefill=0x11)
    oracle.assert_equal(got, exp)
    assert dbuf.guards_intact()


@pytest.mark.parametrize("nsrc,other_off", [(1, 0), (2, 0), (3, 0), (16, 0), (2, 4), (3, 8), (5, 12), (8, 8), (9, 12), (16, 4)])
def test_reduce_copy_in_place_alias(nsrc, other_off):
    """dst == src0 exactly: every element is read before it is written.  With
    the other sources off dst's alignment the unaligned path runs, with the
    aliased source at shift 0."""
    import copy_reduce_amd as tb
    torch = require_gpu()
    n = 300001
    note(f"reduce_copy in-place nsrc={nsrc} n={n} other sources at offset {other_off}")
    srcs = _sources(nsrc, n, seed=5)
    bufs = [DevBuf(torch, n * 4, offset=0 if k == 0 else other_off).upload(s) for k, s in enumerate(srcs)]
    tb.tb_reduce_copy(bufs[0].ptr, [b.ptr for b in bufs], n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    oracle.assert_equal(bufs[0].download().view(np.float32), oracle.ref_reduce(srcs))


def test_torch_api_rejects_strided_tensors():
    """A strided view would be read as if it were contiguous: the torch layer refuses it."""
    torch = require_gpu()
    from copy_reduce_amd.torch_api import reduce_copy
    a = torch.ones(2048, device="cuda")
    dst = torch.zeros(1024, device="cuda")
    with pytest.raises(ValueError):
        reduce_copy(dst, [a[::2]])
    with pytest.raises(ValueError):
        reduce_copy(torch.zeros(2048, device="cuda")[::2], [a[:1024]])
    reduce_copy(dst, [a[:1024], a[1024:]])
    torch.cuda.synchronize()
    assert bool((dst == 2.0).all())


def test_reduce_copy_special_values():
    torch = require_gpu()
    n = 4096
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x80000000, 0x00000000, 0x00000001, 0x807FFFFF, 0x00400000, 0x7F800000,
                         0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7FC00001, 0xFFC12345, 0x7F800001], dtype=np.uint32)
    raw[:specials.size] = specials
    raw[2048:2048 + specials.size] = specials
    a = raw.view(np.float32)
    # N = 1 is a bitwise copy, NaN payloads included
    note("reduce_copy nsrc=1 special values incl. NaN payloads")
    got, exp, _, _ = _run(torch, [a], n)
    assert np.array_equal(got.view(np.uint32), raw)
    # N >= 2 over signed zeros, subnormals, infinities, extremes (no NaN: payloads are not part of the contract)
    finite = np.where(np.isnan(a), np.float32(0.5), a).astype(np.float32)
    b = np.roll(finite, 5)
    c = -np.roll(finite, 11)
    note("reduce_copy nsrc=2,3 special values without NaN")
    for srcs in ([finite, b], [finite, b, c], [c, finite, b]):
        got, exp, _, _ = _run(torch, srcs, n)
        nan_both = np.isnan(got) & np.isnan(exp)
        assert np.array_equal(got.view(np.uint32)[~nan_both], exp.view(np.uint32)[~nan_both])


def test_reduce_copy_fixed_order_worked_examples():
    from conftest import read_golden
    torch = require_gpu()
    for row in read_golden("fp32_order_cases.txt"):
        exp_hex, srcs = row.split(";")
        srcs = [np.full(77, np.uint32(int(h, 16)), dtype=np.uint32).view(np.float32) for h in srcs.split()]
        note(f"reduce_copy worked example {row}")
        got, exp, _, _ = _run(torch, srcs, 77)
        assert np.all(got.view(np.uint32) == np.uint32(int(exp_hex, 16))), row


def test_prep_sources_replicates_slices():
    """validateSource: after prep every slice equals the host reference."""
    from copy_reduce_amd.torch_api import RotatedSources
    torch = require_gpu()
    for nfloats, rot in [(1 << 20, 256 << 20), (1000, 1 << 20), (12345, 100000), (4096, 0)]:
        note(f"prep_sources nfloats={nfloats} R={rot}")
        rs = RotatedSources(2, nfloats, rot, fill=("compress", wl.C3_PCT, 3))
        torch.cuda.synchronize()
        assert rs.k == oracle.num_slices(nfloats * 4, rot)
        for b in range(2):
            ref = oracle.gen_compress(nfloats, b, wl.C3_PCT, 3)
            for s in range(rs.k):
                got = rs.slice_view(b, s).cpu().numpy()
                oracle.assert_equal(got, ref, str((b, s)))


def test_rotation_selects_slice_i_mod_k():
    """Every slice holds the same data in real runs, so validation cannot see a
    rotation bug; here slice s of source b holds PrepSrcValue(s + 16 b, .) instead
    and launch i must return exactly slice ((i mod K) + K) mod K."""
    import copy_reduce_amd as tb
    torch = require_gpu()
    nfloats, rot, nsrc = 4096 + 3, 16 * 4096 * 4, 2
    k = tb.tb_num_slices(nfloats * 4, rot)
    stride = tb.tb_slice_stride(nfloats * 4)
    assert k == 16
    bufs = [torch.empty(k * stride, dtype=torch.uint8, device="cuda") for _ in range(nsrc)]
    for b in range(nsrc):
        for s in range(k):
            data = oracle.gen_default(nfloats, s + 16 * b)
            bufs[b][s * stride:s * stride + nfloats * 4].copy_(torch.from_numpy(data.view(np.uint8).copy()))
    dst = torch.empty(nfloats, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(-3, 2 * k + 1):
        note(f"rotation iteration {i} k={k}")
        ptrs = tb.tb_rotate_sources([int(t.data_ptr()) for t in bufs], stride, k, i)
        tb.tb_reduce_copy(int(dst.data_ptr()), ptrs, nfloats, stream)
        torch.cuda.synchronize()
        s = oracle.slice_of(i, k)
        exp = oracle.ref_reduce([oracle.gen_default(nfloats, s + 16 * b) for b in range(nsrc)])
        oracle.assert_equal(dst.cpu().numpy(), exp, str(i))


def test_reduce_copy_on_side_stream():
    import copy_reduce_amd as tb
    torch = require_gpu()
    n = 1 << 18
    srcs = _sources(3, n, seed=11)
    bufs = [DevBuf(torch, n * 4).upload(s) for s in srcs]
    dst = DevBuf(torch, n * 4)
    side = torch.cuda.Stream()
    note("reduce_copy on a side stream")
    torch.cuda.synchronize()
    tb.tb_reduce_copy(dst.ptr, [b.ptr for b in bufs], n, side.cuda_stream)
    side.synchronize()
    oracle.assert_equal(dst.download().view(np.float32), oracle.ref_reduce(srcs))


def test_reduce_copy_invalid_args_enqueue_nothing():
    import copy_reduce_amd as tb
    torch = require_gpu()
    n = 1024
    dst = DevBuf(torch, n * 4, fill=0x33)
    src = DevBuf(torch, n * 4).upload(oracle.gen_default(n, 0))
    arr = (ctypes.c_void_p * 1)(src.ptr + 2)
    assert tb.lib.tb_reduce_copy(dst.ptr, arr, 1, n, None) == tb.TB_ERR_INVALID
    torch.cuda.synchronize()
    assert np.all(dst.download() == 0x33)


@pytest.mark.parametrize("nsrc", [1, 3])
def test_reduce_copy_captured_in_a_graph_replays_exactly(nsrc):
    """The reduce-copy keeps no state between launches, so it may be captured
    into a HIP graph.  The graph is replayed three times, with the destination
    overwritten eagerly and the device synchronised between replays; every
    replay must give the oracle's bytes."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    n = (1 << 18) + 5
    note(f"reduce_copy graph capture nsrc={nsrc} n={n}")
    srcs = _sources(nsrc, n)
    sbufs = [DevBuf(torch, n * 4, 4 * b).upload(s) for b, s in enumerate(srcs)]
    dbuf = DevBuf(torch, n * 4, 0)
    exp = oracle.ref_reduce(srcs, n=n)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            tb.tb_reduce_copy(dbuf.ptr, [b.ptr for b in sbufs], n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        dbuf.t[dbuf.start:dbuf.start + n * 4].fill_(0x5A + rep)       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dbuf.download().view(np.float32)
        oracle.assert_equal(got, exp, f"replay {rep}")
        assert dbuf.guards_intact()


def test_time_next_launch_events_travel_with_one_launch():
    """tb_time_next_launch: the next launch records the two events itself; the
    launch after it leaves them alone."""
    torch = require_gpu()
    import copy_reduce_amd as tb
    n = 1 << 24                                   # 64 MiB
    note(f"timing hook on a one-source copy n={n}")
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.zeros(n, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    st, sp, ref = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    st.record(s)
    sp.record(s)
    ref.record(s)                                 # later than both first records
    torch.cuda.synchronize()
    tb.tb_time_next_launch(st.cuda_event, sp.cuda_event)
    tb.tb_reduce_copy(int(dst.data_ptr()), [int(src.data_ptr())], n, s.cuda_stream)
    torch.cuda.synchronize()
    assert ref.elapsed_time(st) > 0.0             # both were recorded again, by the launch
    assert ref.elapsed_time(sp) > ref.elapsed_time(st)
    t = st.elapsed_time(sp)
    assert 0.0 < t < 50.0, t
    assert torch.equal(dst, src)
    tb.tb_reduce_copy(int(dst.data_ptr()), [int(src.data_ptr())], n, s.cuda_stream)   # hook consumed
    torch.cuda.synchronize()
    assert st.elapsed_time(sp) == t
