"""CPU tests of libtb_roofs, the measuring instruments of bench.py --roofs: it
loads and exports every symbol include/tb_roofs.h declares, its header is
plain C, its argument checks reject before any HIP call, and the host-side
cut of a batch into tiles covers every copy exactly once."""
import os
import re
import subprocess

import numpy as np

import copy_reduce_amd.roofs as rf
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofs_header_symbols_exported():
    text = open(os.path.join(ROOT, "include", "tb_roofs.h")).read()
    declared = sorted(set(re.findall(r"^(?:int|const char \*)\s*(tbr_\w+)\s*\(", text, re.M)))
    assert declared == sorted(rf.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", rf.ROOFS_LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(declared) <= syms


def test_roofs_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "tb_roofs.h"\nint main(void){tbr_tile t = {0, 0, 16, 0}; (void)t;'
                   ' return tbr_read(0, 0, 0, 0) == TBR_ERR_INVALID ? 0 : 1;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-c", str(src), "-o", str(tmp_path / "use.o")], check=True)


def test_roofs_argument_checks():
    lib = rf.lib
    bufs = rf._ptrs([0x1000])
    assert lib.tbr_read(None, 1, 4096, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_read(bufs, 0, 4096, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_read(bufs, 18, 4096, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_read(rf._ptrs([0x1008]), 1, 4096, None) == rf.TBR_ERR_INVALID      # misaligned
    assert lib.tbr_read(bufs, 1, 4100, None) == rf.TBR_ERR_INVALID                     # not a multiple of 16
    assert lib.tbr_read(bufs, 1, 0, None) == rf.TBR_OK
    assert lib.tbr_write(bufs, 1, 4096, 0, 3, None) == rf.TBR_ERR_INVALID               # unknown policy
    two = rf._ptrs([0x1000, 0x3000])
    assert lib.tbr_combine(two, 2, 0x5000, 4096, 3, None) == rf.TBR_ERR_INVALID          # unknown policy
    assert lib.tbr_combine(two, 2, 0x3800, 4096, 0, None) == rf.TBR_ERR_INVALID          # dst overlaps a source
    assert lib.tbr_combine(two, 2, 0x5008, 4096, 0, None) == rf.TBR_ERR_INVALID          # misaligned dst
    assert lib.tbr_combine(two, 2, None, 4096, 0, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_combine(two, 0, 0x5000, 4096, 0, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_combine(rf._ptrs([0x1000] * 17), 17, 0x90000, 4096, 0, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_combine(two, 2, 0x5000, 4100, 0, None) == rf.TBR_ERR_INVALID          # not a multiple of 16
    assert lib.tbr_combine(two, 2, 0x5000, 0, 2, None) == rf.TBR_OK
    assert lib.tbr_copy(0x1800, 0x1000, 4096, 0, None) == rf.TBR_ERR_INVALID            # overlapping
    assert lib.tbr_copy(0x2000, 0x1008, 16, 0, None) == rf.TBR_ERR_INVALID              # misaligned
    assert lib.tbr_copy(0x2000, 0x1000, 0, 0, None) == rf.TBR_OK
    assert lib.tbr_tiles_copy(None, 5, 0, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_tiles_copy(0x1004, 5, 0, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_tiles_write(0x1000, 5, 0, 7, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_tiles_copy(0x1000, 5, 3, None) == rf.TBR_ERR_INVALID
    assert lib.tbr_tiles_read(None, 0, None) == rf.TBR_OK


def test_cut_tiles_covers_every_copy_exactly():
    rng = np.random.default_rng(3)
    n = 500
    sizes = (rng.integers(1, 1200, size=n) * 16).astype(np.uint64)
    src = np.cumsum(np.concatenate([[0], sizes[:-1]])).astype(np.uint64)
    dst = (rng.permutation(n).astype(np.uint64) * np.uint64(32768))
    desc = np.stack([src, dst, sizes], axis=1)
    t = rf.cut_tiles(desc, 1 << 32, 1 << 36)
    assert int(t[:, 2].sum()) == int(sizes.sum())
    assert np.all((t[:, 2] >= 16) & (t[:, 2] <= 4096) & (t[:, 2] % 16 == 0))
    # every byte of every copy is covered once, in order
    k = 0
    for s, d, b in desc.astype(np.int64):
        off = 0
        while off < b:
            assert (int(t[k, 0]), int(t[k, 1]), int(t[k, 2])) == ((1 << 32) + s + off, (1 << 36) + d + off,
                                                                 min(4096, b - off))
            off += 4096
            k += 1
    assert k == t.shape[0]


def test_cut_tiles_of_c4_match_its_bytes():
    b = wl.batch_c4(with_payload=False)
    t = rf.cut_tiles(b.desc, 0, 0)
    assert int(t[:, 2].sum()) == b.total_bytes
    assert t.shape[0] == int(((b.desc[:, 2].astype(np.int64) + 4095) // 4096).sum())
