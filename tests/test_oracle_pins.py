"""Pins for the CPU oracle: things the pages and the mathematics fix, checked
without re-running the oracle's own formulas.  CPU only."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from conftest import read_golden

MiB = 1 << 20


# --------------------------------------------------------------------------
# Slice count K and slice stride (PR #365, Technical Details / Test Result)
# --------------------------------------------------------------------------

def test_slice_counts_printed_on_page():
    for row in read_golden("slice_counts.txt"):
        nbytes, rot, k, alloc = map(int, row.split())
        assert oracle.num_slices(nbytes, rot) == k
        assert k * oracle.slice_stride(nbytes) == alloc


def test_slice_count_edge_cases():
    assert oracle.num_slices(4 * MiB, 0) == 1          # 0 disables rotation
    assert oracle.num_slices(0, 256 * MiB) == 1        # nothing to replicate
    assert oracle.num_slices(512 * MiB, 256 * MiB) == 1
    assert oracle.num_slices(1, 2**64 - 1) == 2**64 - 1  # no overflow in the ceiling


def test_slice_count_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        n = int(rng.integers(1, 1 << 40))
        r = int(rng.integers(1, 1 << 40))
        # smallest K with K * n >= r, found by searching around r // n
        k = max(1, r // n)
        while k * n < r:
            k += 1
        assert oracle.num_slices(n, r) == k


@pytest.mark.parametrize("nbytes,expected", [(0, 0), (1, 256), (255, 256), (256, 256), (257, 512),
                                             (4 * MiB, 4 * MiB), (4 * MiB + 4, 4 * MiB + 256)])
def test_slice_stride_rounds_to_256(nbytes, expected):
    assert oracle.slice_stride(nbytes) == expected


# Configurations' K values (SRC_ROTATE_BYTES = 256 MiB unless stated)
@pytest.mark.parametrize("nbytes,rot,k", [
    (4 * MiB, 256 * MiB, 64), (256 * MiB, 256 * MiB, 1), (256 * MiB, 0, 1), (64 * MiB, 256 * MiB, 4),
    (8 * MiB, 256 * MiB, 32), (16 * MiB, 256 * MiB, 16), (32 * MiB, 256 * MiB, 8),
    (128 * MiB, 256 * MiB, 2), (512 * MiB, 256 * MiB, 1)])
def test_config_slice_counts(nbytes, rot, k):
    assert oracle.num_slices(nbytes, rot) == k


def test_slice_of_folds_negative_iterations():
    # K = 64 with 3 warmups (-3..-1) and 10 timed iterations (0..9)
    assert [oracle.slice_of(i, 64) for i in range(-3, 10)] == [61, 62, 63] + list(range(10))
    for k in (1, 2, 3, 7, 64):
        for i in range(-3 * k, 3 * k):
            s = oracle.slice_of(i, k)
            assert 0 <= s < k
            assert (i - s) % k == 0     # same residue class, any sign convention


# --------------------------------------------------------------------------
# Default source pattern ("Expected source pattern", PrepSrcValue)
# --------------------------------------------------------------------------

def test_prep_src_values_worked_by_hand():
    for row in read_golden("prep_src_values.txt"):
        b, i, v = map(int, row.split())
        got = oracle.gen_default(i + 1, b)[i]
        assert got == np.float32(v), (b, i, got, v)


def test_prep_src_pattern_structure():
    v0 = oracle.gen_default(3 * 383 + 17, 0).astype(np.int64)
    # period 383
    assert np.array_equal(v0[383:766], v0[:383]) and np.array_equal(v0[766:1149], v0[:383])
    # 517 = 134 (mod 383) and 383 is prime, so one period is a permutation of 31..413
    assert sorted(v0[:383].tolist()) == list(range(31, 414))
    assert int(v0[:383].sum()) == sum(range(31, 414)) == 85026
    # buffer b is buffer 0 scaled by b + 1
    for b in (1, 2, 5, 15):
        vb = oracle.gen_default(1000, b).astype(np.int64)
        assert np.array_equal(vb, (b + 1) * v0[:1000])


def test_fill_pattern_repeats():
    pat = np.array([1.5, -2.25, 3.0], dtype=np.float32)
    out = oracle.gen_pattern(10, pat)
    assert out.tolist() == [1.5, -2.25, 3.0] * 3 + [1.5]


# --------------------------------------------------------------------------
# fillCompress (reading: SplitMix64 streams, leading-byte zeroing)
# --------------------------------------------------------------------------

def test_splitmix64_published_outputs():
    for row in read_golden("splitmix64.txt"):
        seed, j, v = map(int, row.split())
        assert oracle.splitmix64(seed, j) == v


def test_compress_values_on_grid_and_in_range():
    x = oracle.gen_compress(1 << 16, 0, (100, 0, 0, 0, 0), 3)
    assert x.min() >= -1.0 and x.max() < 1.0
    scaled = x.astype(np.float64) * 2**23
    assert np.array_equal(scaled, np.rint(scaled))
    # the value of float i is drawn from output i of the value stream: check a few
    # directly from the published generator (value key = seed ^ 2b)
    for i in (0, 1, 17, 1000):
        u = oracle.splitmix64(3 ^ 0, i) >> 40
        assert x[i] == np.float32((u - 2**23) / 2**23)


@pytest.mark.parametrize("cat,zero_bytes", [(1, 1), (2, 2), (3, 4), (4, 32)])
def test_compress_category_zeroes_leading_bytes(cat, zero_bytes):
    pct = [0] * 5
    pct[cat] = 100
    n = 16 * 1000 + 5              # partial last line
    x = oracle.gen_compress(n, 2, pct, 11)
    full = oracle.gen_compress(n, 2, (100, 0, 0, 0, 0), 11)
    xb = x.view(np.uint8)
    fb = full.view(np.uint8)
    for line in range(0, len(xb), 64):
        seg, ref = xb[line:line + 64], fb[line:line + 64]
        z = min(zero_bytes, len(seg))
        assert not seg[:z].any()
        assert np.array_equal(seg[z:], ref[z:])


def test_compress_category_frequencies():
    n = 16 * (1 << 20)           # 1,048,576 lines, the size of one C3 buffer
    pct = np.array(wl.C3_PCT)
    for b in range(4):
        x = oracle.gen_compress(n, b, wl.C3_PCT, wl.C3_SEED).view(np.uint8).reshape(-1, 64)
        lead32 = ~x[:, :32].any(axis=1)
        lead4 = ~x[:, :4].any(axis=1)
        nlines = x.shape[0]
        # lines whose first 32 bytes are all zero: the 32B0 category (random ones never are)
        exp = pct[4] / 100 * nlines
        sd = math.sqrt(nlines * pct[4] / 100 * (1 - pct[4] / 100))
        assert abs(lead32.sum() - exp) < 5 * sd
        # first 4 bytes zero: 4B0 + 32B0 (random/1B0/2B0 with a zero low float are ~2^-24 rare)
        exp4 = (pct[3] + pct[4]) / 100 * nlines
        sd4 = math.sqrt(nlines * (pct[3] + pct[4]) / 100)
        assert abs(lead4.sum() - exp4) < 5 * sd4


def test_compress_rejects_bad_percentages():
    with pytest.raises(ValueError):
        oracle.gen_compress(16, 0, (50, 20, 10, 10, 5), 1)


def test_compress_buffers_differ_and_seeds_matter():
    a = oracle.gen_compress(4096, 0, wl.C3_PCT, 3)
    b = oracle.gen_compress(4096, 1, wl.C3_PCT, 3)
    c = oracle.gen_compress(4096, 0, wl.C3_PCT, 4)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


# --------------------------------------------------------------------------
# Expected destination (dstReference)
# --------------------------------------------------------------------------

def _bits(hexstr):
    return np.array([int(hexstr, 16)], dtype=np.uint32).view(np.float32)[0]


def test_reduce_worked_examples_fixed_order():
    for row in read_golden("fp32_order_cases.txt"):
        exp, srcs = row.split(";")
        sources = [np.array([_bits(h)] * 3, dtype=np.float32) for h in srcs.split()]
        got = oracle.ref_reduce(sources)
        assert np.all(got.view(np.uint32) == np.uint32(int(exp, 16))), row


@pytest.mark.parametrize("nsrc", [1, 2, 3, 4, 8, 16])
def test_reduce_default_pattern_closed_form(nsrc):
    # buffer b holds (b + 1) * v(i); the sum is v(i) * N (N + 1) / 2 exactly (< 2^24)
    n = 5000
    srcs = [oracle.gen_default(n, b) for b in range(nsrc)]
    v = oracle.gen_default(n, 0).astype(np.int64)
    expected = (v * (nsrc * (nsrc + 1) // 2)).astype(np.float32)
    oracle.assert_equal(oracle.ref_reduce(srcs), expected)


def test_reduce_zero_sources_is_memset():
    out = oracle.ref_reduce([], n=37)
    assert not out.view(np.uint8).any()
    out = oracle.ref_reduce([], n=37, memset_byte=0xAB)
    assert np.all(out.view(np.uint8) == 0xAB)


def test_reduce_one_source_is_bitwise_copy():
    raw = np.random.default_rng(1).integers(0, 2**32, size=4096, dtype=np.uint64).astype(np.uint32)
    raw[:8] = [0x7FC00001, 0xFFC12345, 0x7F800001, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F800000, 0]
    src = raw.view(np.float32)
    out = oracle.ref_reduce([src])
    assert np.array_equal(out.view(np.uint32), raw)


def test_reduce_each_step_correctly_rounded():
    """dstReference[k] = RNE(dstReference[k-1] + srcReference[k-1]): the sum of two
    binary32 values on the 2^-23 grid is exact in binary64, and converting that
    exact value to binary32 is the correctly rounded result."""
    n = 1 << 16
    srcs = [oracle.gen_compress(n, b, wl.C3_PCT, 7) for b in range(4)]
    prev = oracle.ref_reduce(srcs[:1])
    for k in range(2, 5):
        cur = oracle.ref_reduce(srcs[:k])
        exact = prev.astype(np.float64) + srcs[k - 1].astype(np.float64)
        oracle.assert_equal(cur, exact.astype(np.float32))
        prev = cur


def test_reduce_within_rounding_bound_of_exact_sum():
    n = 1 << 16
    srcs = [oracle.gen_compress(n, b, wl.C3_PCT, 9) for b in range(4)]
    exact = sum(s.astype(np.float64) for s in srcs)        # exact: < 4 in size, 2^-23 grid
    got = oracle.ref_reduce(srcs).astype(np.float64)
    # three roundings, each at most half an ulp of a partial sum below 4 (2^-22 / 2)
    assert np.max(np.abs(got - exact)) <= 3 * 2.0**-23
    assert np.mean(got == exact) > 0.9


def test_reduce_order_is_observable_on_compress_sources():
    """A pairwise order (s0+s1)+(s2+s3) must differ from left to right on some
    elements, so parity on these sources detects a reordered sum."""
    n = 1 << 18
    srcs = [oracle.gen_compress(n, b, wl.C3_PCT, wl.C3_SEED) for b in range(4)]
    left = oracle.ref_reduce(srcs)
    pair = oracle.ref_reduce([oracle.ref_reduce(srcs[:2]), oracle.ref_reduce(srcs[2:])])
    frac = np.mean(left.view(np.uint32) != pair.view(np.uint32))
    assert 0.001 < frac < 0.05


# --------------------------------------------------------------------------
# Batched copy (Mooncake RFC #5041, Design of #5040)
# --------------------------------------------------------------------------

def test_batch_brute_force_tiny():
    rng = np.random.default_rng(5)
    for trial in range(30):
        b = wl.batch_random(seed=trial, n=int(rng.integers(0, 12)), max_bytes=300, pool_bytes=1 << 14)
        pool = np.full(b.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
        ref = bytearray(pool.tobytes())
        payload = b.payload.tobytes()
        for s, d, nb in b.desc.tolist():
            for j in range(nb):                      # byte by byte, pure Python
                ref[d + j] = payload[s + j]
        oracle.ref_batch(pool, b.payload, b.desc)
        assert pool.tobytes() == bytes(ref)


def test_batch_untouched_bytes_and_empty_batch():
    b = wl.batch_random(seed=99, n=40, max_bytes=500, pool_bytes=1 << 16)
    pool = np.full(b.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    oracle.ref_batch(pool, b.payload, b.desc[:0])
    assert np.all(pool == wl.POOL_FILL)
    oracle.ref_batch(pool, b.payload, b.desc)
    written = np.zeros(b.pool_bytes, dtype=bool)
    for s, d, nb in b.desc.tolist():
        written[d:d + nb] = True
        assert np.array_equal(pool[d:d + nb], b.payload[s:s + nb])
    assert np.all(pool[~written] == wl.POOL_FILL)


def test_c4_c5_shapes():
    c4 = wl.batch_c4(with_payload=False)
    assert c4.ncopies == 47_520
    sizes = c4.desc[:, 2].astype(np.int64)
    assert sizes.min() >= 64 and sizes.max() <= 16384 and np.all(sizes % 64 == 0)
    assert len(np.unique(c4.desc[:, 1])) == c4.ncopies and np.all(c4.desc[:, 1] % 16384 == 0)
    # log-uniform: about half the copies are at most 1 KiB
    assert 0.45 < np.mean(sizes <= 1024) < 0.55
    c5 = wl.batch_c5(with_payload=False)
    assert c5.ncopies == 11_044
    s5 = c5.desc[:, 2].astype(np.int64)
    assert (s5 == 8 * MiB).sum() == 4 and (s5 == 2112).sum() >= 3840   # the log-uniform part can draw 2,112 too
    # destinations disjoint
    order = np.argsort(c5.desc[:, 1])
    d, s = c5.desc[order, 1].astype(np.int64), s5[order]
    assert np.all(d[:-1] + s[:-1] <= d[1:])
    assert int(d[-1] + s[-1]) <= c5.pool_bytes


def test_batch_preconditions_hold_and_are_checked():
    """Every workload satisfies the batched copy's preconditions (disjoint,
    in-range destinations), and the check rejects a batch that does not."""
    for b in (wl.batch_c4(with_payload=False), wl.batch_c5(with_payload=False),
              wl.batch_random(3, 500, max_bytes=5000, pool_bytes=8 << 20)):
        assert b.check() is b
    bad = wl.batch_random(4, 10, max_bytes=100, pool_bytes=1 << 16, min_bytes=8)
    bad.desc[1, 1] = bad.desc[0, 1] + 1                      # overlaps copy 0
    with pytest.raises(ValueError):
        bad.check()
    far = wl.batch_random(5, 10, max_bytes=100, pool_bytes=1 << 16, min_bytes=8)
    far.desc[0, 1] = far.pool_bytes                          # past the pool
    with pytest.raises(ValueError):
        far.check()



def test_c4_placements_keep_the_copies_and_move_only_destinations():
    """The destination-placement study's batches: C4's sizes (as a multiset),
    sources packed in descriptor order, valid disjoint destinations, and the
    placement each one names."""
    c4 = wl.batch_c4(with_payload=False)
    ref_sizes = np.sort(c4.desc[:, 2])
    for p in wl.C4_PLACEMENTS:
        b = wl.batch_c4_placed(p).check()
        d = b.desc.astype(np.int64)
        assert b.ncopies == c4.ncopies and np.array_equal(np.sort(b.desc[:, 2]), ref_sizes)
        assert d[0, 0] == 0 and np.all(d[1:, 0] == d[:-1, 0] + d[:-1, 2])      # one source stream
        assert len(b.payload) == b.src_bytes
        if p == "random_slots":
            assert np.array_equal(b.desc, c4.desc)
        elif p == "random_slots_sorted":
            assert np.all(np.diff(d[:, 1]) > 0)
            assert np.array_equal(np.sort(d[:, 1]), np.sort(c4.desc[:, 1].astype(np.int64)))
        elif p == "consecutive_slots":
            assert np.array_equal(d[:, 1], np.arange(b.ncopies) * wl.SLOT_BYTES)
        elif p == "packed":
            assert np.array_equal(d[:, 1], d[:, 0])
        else:
            assert int((d[:, 1] + d[:, 2]).max()) == b.total_bytes              # dense ...
            assert not np.all(np.diff(d[:, 1]) > 0)                            # ... visited out of order
    with pytest.raises(ValueError):
        wl.batch_c4_placed("diagonal")

# --------------------------------------------------------------------------
# Comparator ("How validation (ValidateAllTransfers) works")
# --------------------------------------------------------------------------

@pytest.mark.parametrize("where", [0, 12345, 99999])
def test_mismatch_report_names_index_expected_and_actual(where):
    """A failure names the first differing element with its expected and
    actual values: a planted float and a planted byte are reported exactly."""
    exp = oracle.gen_default(100000, 1)
    assert oracle.mismatch_report(exp.copy(), exp) is None
    out = exp.copy()
    out[where] = np.float32(-0.375)
    if where + 7 < out.size:
        out[where + 7] = np.float32(1e30)                 # a later difference is not the one reported
    i, e, a = oracle.mismatch_report(out, exp)
    assert (i, e.view(np.uint32), a.view(np.uint32)) == (where, exp[where].view(np.uint32),
                                                        np.float32(-0.375).view(np.uint32))
    with pytest.raises(AssertionError, match=f"element {where}: expected {float(exp[where])!r} .* got -0.375"):
        oracle.assert_equal(out, exp)
    pool = np.full(4096, 0xA5, np.uint8)
    bad = pool.copy()
    bad[where % 4096] = 0x3C
    assert oracle.mismatch_report(bad, pool) == (where % 4096, 0xA5, 0x3C)


@pytest.mark.parametrize("where", [0, 12345, 99999])
def test_first_mismatch_reports_corrupted_index(where):
    exp = oracle.gen_default(100000, 0)
    out = exp.copy()
    oracle.assert_equal(out, exp)
    out.view(np.uint8)[where * 4 + 2] ^= 0x40
    assert oracle.first_mismatch(out, exp) == where
    bout, bexp = out.view(np.uint8), exp.view(np.uint8)
    assert oracle.first_mismatch(bout, bexp) == where * 4 + 2
