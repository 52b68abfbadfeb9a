"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds none of the method's arithmetic: no source pattern, no sum,
no copy.  It only draws the *inputs* of the batched-copy workloads (descriptor
lists and random payload bytes) and names the workload parameters, so that the
tests and the benchmark can hand the very same arrays to the oracle and to the
GPU library.  The reduce-copy source patterns are part of the method
(PrepareReference) and are generated independently by each side.

Descriptor lists are (src_offset, dst_offset, bytes) triples, uint64, shape
(n, 3): offsets into a contiguous source image and into a destination pool.
The caller adds device base addresses to turn them into tb_copy_desc records.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

KiB = 1024
MiB = 1024 * KiB
GiB = 1024 * MiB

DEFAULT_ROTATE_BYTES = 256 * MiB      # SRC_ROTATE_BYTES default (PR #365)
POOL_BYTES = 4 * GiB                  # destination pool of the batched workloads
SLOT_BYTES = 16 * KiB                 # destination slot granularity in the pool
POOL_FILL = 0xA5                      # pre-fill byte: never-written bytes keep it


# --------------------------------------------------------------------------
# Reduce-copy workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class ReduceWorkload:
    name: str
    nsrc: int
    nfloats: int
    rotate_bytes: int
    fill: Optional[tuple] = None        # None = default PrepSrcValue pattern
    warmup: int = 3
    iters: int = 10

    @property
    def num_bytes(self) -> int:
        return self.nfloats * 4

    @property
    def algorithmic_bytes(self) -> int:
        """(N + 1) x numBytes per launch; numBytes for a memset (N = 0)."""
        return (self.nsrc + 1) * self.num_bytes if self.nsrc > 0 else self.num_bytes


C3_PCT = (50, 20, 10, 10, 10)          # random, 1B0, 2B0, 4B0, 32B0
C3_SEED = 3

REDUCE_CONFIGS = {
    # single-source copy, 4 MiB, rotation on (K = 64)
    "c1_copy_4MiB_rot": ReduceWorkload("c1_copy_4MiB_rot", 1, 1 << 20, DEFAULT_ROTATE_BYTES),
    "c1_copy_4MiB_norot": ReduceWorkload("c1_copy_4MiB_norot", 1, 1 << 20, 0),
    # two-source reduce, 256 MiB per buffer, rotation on (K = 1) and the R = 0 control
    "c2_reduce2_256MiB_rot": ReduceWorkload("c2_reduce2_256MiB_rot", 2, 64 << 20, DEFAULT_ROTATE_BYTES),
    "c2_reduce2_256MiB_norot": ReduceWorkload("c2_reduce2_256MiB_norot", 2, 64 << 20, 0),
    # four-source reduce, 64 MiB per buffer, fillCompress sources, K = 4
    "c3_reduce4_64MiB_compress": ReduceWorkload(
        "c3_reduce4_64MiB_compress", 4, 16 << 20, DEFAULT_ROTATE_BYTES,
        fill=("compress", C3_PCT, C3_SEED)),
}

SWEEP_BYTES = [8 * MiB, 16 * MiB, 32 * MiB, 64 * MiB, 128 * MiB, 256 * MiB, 512 * MiB]


def sweep_workload(num_bytes: int, rotate: bool) -> ReduceWorkload:
    tag = "rot" if rotate else "norot"
    return ReduceWorkload(f"c5_sweep_{num_bytes // MiB}MiB_{tag}", 1, num_bytes // 4,
                          DEFAULT_ROTATE_BYTES if rotate else 0)


# --------------------------------------------------------------------------
# Batched-copy workloads
# --------------------------------------------------------------------------

@dataclass
class Batch:
    """One descriptor array plus the bytes its sources hold."""
    name: str
    desc: np.ndarray                   # (n, 3) uint64: src_off, dst_off, bytes
    src_bytes: int                     # size of the contiguous source image
    pool_bytes: int
    seed: int
    payload: Optional[np.ndarray] = field(default=None, repr=False)

    @property
    def ncopies(self) -> int:
        return int(self.desc.shape[0])

    @property
    def total_bytes(self) -> int:
        return int(self.desc[:, 2].sum()) if self.ncopies else 0

    @property
    def algorithmic_bytes(self) -> int:
        """Read plus write of every payload byte: 2 x sum(bytes)."""
        return 2 * self.total_bytes

    def check(self) -> "Batch":
        """Preconditions the batched copy assumes and cannot check on the
        device: every source range inside the source image, every destination
        range inside the pool, destination ranges pairwise disjoint.  Raises
        ValueError; returns self."""
        d = self.desc.astype(np.uint64)
        if d.ndim != 2 or d.shape[1] != 3:
            raise ValueError("descriptors must be an (n, 3) array")
        s, t, b = (d[:, k].astype(object) for k in range(3))   # exact integers
        if any(x + y > self.src_bytes for x, y in zip(s, b)):
            raise ValueError("a source range lies outside the source image")
        if any(x + y > self.pool_bytes for x, y in zip(t, b)):
            raise ValueError("a destination range lies outside the pool")
        live = np.flatnonzero(d[:, 2] > 0)
        order = live[np.argsort(d[live, 1], kind="stable")]
        ends = d[order, 1] + d[order, 2]
        if np.any(ends[:-1] > d[order[1:], 1]):
            raise ValueError("destination ranges overlap")
        return self


def log_uniform_sizes(rng: np.random.Generator, n: int, lo: int, hi: int,
                      granule: int = 64) -> np.ndarray:
    """Sizes log-uniform over [lo, hi], rounded to multiples of `granule`."""
    u = rng.random(n)
    x = np.exp2(np.log2(lo / granule) + u * np.log2(hi / lo))
    sizes = granule * np.rint(x).astype(np.int64)
    return np.clip(sizes, lo, hi).astype(np.uint64)


def _pack_sources(sizes: np.ndarray, align: int = 16) -> Tuple[np.ndarray, int]:
    """Contiguous source offsets in descriptor order (each rounded up to `align`)."""
    padded = (sizes.astype(np.int64) + align - 1) // align * align
    offs = np.zeros(len(sizes), dtype=np.int64)
    if len(sizes) > 1:
        offs[1:] = np.cumsum(padded[:-1])
    total = int(padded.sum()) if len(sizes) else 0
    return offs.astype(np.uint64), total


def random_payload(rng: np.random.Generator, nbytes: int) -> np.ndarray:
    return rng.integers(0, 256, size=nbytes, dtype=np.uint8)


def batch_c4(seed: int = 4, n: int = 47_520, pool_bytes: int = POOL_BYTES,
             with_payload: bool = True) -> Batch:
    """Head-sliced KV shape: n copies, log-uniform 64 B - 16 KiB (x 64 B),
    contiguous sources, destinations in distinct random 16 KiB slots."""
    rng = np.random.default_rng(seed)
    sizes = log_uniform_sizes(rng, n, 64, 16 * KiB)
    nslots = pool_bytes // SLOT_BYTES
    slots = rng.choice(nslots, size=n, replace=False).astype(np.uint64)
    src_off, src_total = _pack_sources(sizes)
    desc = np.stack([src_off, slots * np.uint64(SLOT_BYTES), sizes], axis=1).astype(np.uint64)
    b = Batch("c4_scatter_47520", desc, src_total, pool_bytes, seed)
    if with_payload:
        b.payload = random_payload(rng, src_total)
    return b


def batch_c5(seed: int = 5, pool_bytes: int = POOL_BYTES, with_payload: bool = True,
             n_block: int = 7_200, n_index: int = 3_840, n_mla: int = 4) -> Batch:
    """Mixed KV batch: n_block copies log-uniform 512 B - 16 KiB (x 64 B),
    n_index copies of 2,112 B and n_mla copies of 8 MiB, one shuffled array.
    The 8 MiB copies land in distinct 8 MiB-aligned regions; the others in
    distinct 16 KiB slots outside those regions."""
    rng = np.random.default_rng(seed)
    small = log_uniform_sizes(rng, n_block, 512, 16 * KiB)
    index = np.full(n_index, 2112, dtype=np.uint64)
    mla = np.full(n_mla, 8 * MiB, dtype=np.uint64)

    nregions = pool_bytes // (8 * MiB)
    regions = rng.choice(nregions, size=n_mla, replace=False).astype(np.uint64)
    slots_per_region = (8 * MiB) // SLOT_BYTES
    nslots = pool_bytes // SLOT_BYTES
    taken = np.zeros(nslots, dtype=bool)
    for r in regions:
        taken[int(r) * slots_per_region:(int(r) + 1) * slots_per_region] = True
    free = np.flatnonzero(~taken)
    nsmall = n_block + n_index
    small_slots = rng.choice(free, size=nsmall, replace=False).astype(np.uint64)

    sizes = np.concatenate([small, index, mla])
    dst = np.concatenate([small_slots * np.uint64(SLOT_BYTES), regions * np.uint64(8 * MiB)])
    order = rng.permutation(len(sizes))
    sizes = sizes[order]
    dst = dst[order]
    src_off, src_total = _pack_sources(sizes)
    desc = np.stack([src_off, dst, sizes], axis=1).astype(np.uint64)
    b = Batch("c5_mixed_kv_11044", desc, src_total, pool_bytes, seed)
    if with_payload:
        b.payload = random_payload(rng, src_total)
    return b


def batch_random(seed: int, n: int, max_bytes: int, pool_bytes: int,
                 src_align: int = 1, dst_align: int = 1, size_align: int = 1,
                 min_bytes: int = 0) -> Batch:
    """Small random batches for parity tests: arbitrary sizes and alignments,
    destinations disjoint (laid out in a shuffled order with random gaps)."""
    rng = np.random.default_rng(seed)
    sizes = rng.integers(min_bytes, max_bytes + 1, size=n).astype(np.int64)
    sizes = sizes // size_align * size_align
    # sources: packed with random misalignment
    src_off = np.zeros(n, dtype=np.int64)
    pos = 0
    for i in range(n):
        pos = (pos + src_align - 1) // src_align * src_align + int(rng.integers(0, 64)) * src_align
        src_off[i] = pos
        pos += int(sizes[i])
    src_total = pos + 64
    # destinations: disjoint ranges in a random order with random gaps
    order = rng.permutation(n)
    dst_off = np.zeros(n, dtype=np.int64)
    pos = int(rng.integers(0, 64)) * dst_align
    for i in order:
        pos = (pos + dst_align - 1) // dst_align * dst_align
        dst_off[i] = pos
        pos += int(sizes[i]) + int(rng.integers(0, 48)) * dst_align
    if pos > pool_bytes:
        raise ValueError("pool too small for this random batch")
    desc = np.stack([src_off, dst_off, sizes], axis=1).astype(np.uint64)
    b = Batch(f"random_{seed}", desc, src_total, pool_bytes, seed)
    b.payload = random_payload(rng, src_total)
    return b



C4_PLACEMENTS = ("random_slots", "random_slots_sorted", "consecutive_slots", "packed", "packed_shuffled")


def batch_c4_placed(placement: str, seed: int = 4, pool_bytes: int = POOL_BYTES) -> Batch:
    """C4's copies (the same sizes) under another destination placement, for
    telling what the destination pattern costs.  Sources are always packed in
    descriptor order, so the reads stay one stream and only the writes change:
      random_slots         C4 itself: distinct random 16 KiB slots, in drawing order
      random_slots_sorted  the same slots, descriptors in increasing destination order
      consecutive_slots    descriptor k in slot k (every slot used, in order)
      packed               destinations adjacent in descriptor order, like the sources
      packed_shuffled      the packed destinations, descriptors in a random order."""
    base = batch_c4(seed=seed, pool_bytes=pool_bytes, with_payload=True)
    sizes = base.desc[:, 2].copy()
    dst = base.desc[:, 1].copy()
    n = len(sizes)
    if placement == "random_slots":
        order = np.arange(n)
    elif placement == "random_slots_sorted":
        order = np.argsort(dst, kind="stable")
    elif placement in ("consecutive_slots", "packed"):
        order = np.arange(n)
    elif placement == "packed_shuffled":
        order = np.random.default_rng(seed + 1000).permutation(n)
    else:
        raise ValueError(f"unknown placement {placement!r}")
    sizes, dst = sizes[order], dst[order]
    if placement == "consecutive_slots":
        dst = np.arange(n, dtype=np.uint64) * np.uint64(SLOT_BYTES)
    elif placement in ("packed", "packed_shuffled"):
        packed, _ = _pack_sources(base.desc[:, 2])       # adjacent, in C4's drawing order
        dst = packed[order]
    src_off, src_total = _pack_sources(sizes)
    desc = np.stack([src_off, dst, sizes], axis=1).astype(np.uint64)
    return Batch(f"c4_{placement}", desc, src_total, pool_bytes, seed, payload=base.payload[:src_total])
