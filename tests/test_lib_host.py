"""CPU tests of libtb's host half: the library loads and exports every symbol
include/tb.h declares, and its host-only logic (slice geometry, rotation,
PrepareReference generators, argument checks) agrees with the oracle.
No GPU work is enqueued here: the argument checks reject before any HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import copy_reduce_amd as tb
import oracle
import workloads as wl
from copy_reduce_amd import _tb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MiB = 1 << 20


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "tb.h")).read()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*(tb_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    declared = _declared_symbols()
    assert len(declared) == len(_tb.EXPORTS) and sorted(_tb.EXPORTS) == declared
    for name in declared:
        assert hasattr(tb.lib, name)
    # and they are real dynamic symbols of the shared object
    out = subprocess.run(["nm", "-D", "--defined-only", tb.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(declared) <= syms


def test_c_consumer_check_builds(tmp_path):
    """The plain-C program the GPU tests run compiles and links against
    libtb.so and the HIP runtime (gcc, C11, warnings as errors)."""
    import importlib.util
    import shutil
    spec = importlib.util.spec_from_file_location("_capi_build", os.path.join(ROOT, "tests", "capi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if not os.path.exists(os.path.join(ROOT, "copy_reduce_amd", "libtb.so")):
        pytest.skip("libtb.so not built")
    here = tmp_path / "capi"
    here.mkdir()
    shutil.copy(os.path.join(ROOT, "tests", "capi", "capi_check.c"), here)
    mod.HERE, mod.OUT = str(here), str(here / "capi_check")
    out = mod.build()
    assert os.access(out, os.X_OK)


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "tb.h"\nint main(void){uint64_t k; return tb_num_slices(1,2,&k);}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-c", str(src), "-o", str(tmp_path / "use.o")], check=True)


def test_status_strings():
    for st in (0, -1, -2, -3, -4, 7):
        assert isinstance(tb.tb_status_string(st), str) and tb.tb_status_string(st)


@pytest.mark.parametrize("nbytes,rot", [(4 * MiB, 256 * MiB), (256 * MiB, 256 * MiB), (256 * MiB, 0),
                                        (64 * MiB, 256 * MiB), (0, 256 * MiB), (3, 10), (10, 3), (1, 2**64 - 1)])
def test_num_slices_matches_oracle(nbytes, rot):
    assert tb.tb_num_slices(nbytes, rot) == oracle.num_slices(nbytes, rot)


def test_num_slices_random_vs_oracle():
    rng = np.random.default_rng(1)
    for _ in range(3000):
        n, r = int(rng.integers(0, 1 << 34)), int(rng.integers(0, 1 << 34))
        assert tb.tb_num_slices(n, r) == oracle.num_slices(n, r)
        assert tb.tb_slice_stride(n) == oracle.slice_stride(n)


def test_rotation_matches_oracle_slice_of():
    bases = [0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0100]
    for k in (1, 2, 4, 64):
        stride = 4 * MiB
        for i in range(-3 * k, 3 * k + 1):
            got = tb.tb_rotate_sources(bases, stride, k, i)
            s = oracle.slice_of(i, k)
            assert got == [b + s * stride for b in bases]


def test_rotation_rejects_bad_args():
    with pytest.raises(tb.TBError):
        tb.tb_rotate_sources([0x1000], 256, 0, 1)           # k == 0
    with pytest.raises(tb.TBError):
        tb.tb_rotate_sources([0x1000] * 17, 256, 4, 1)      # more than TB_MAX_SRCS
    with pytest.raises(tb.TBError):
        tb.tb_rotate_sources([2**64 - 16], 2**40, 4, 3)     # address overflow


def _lib_gen(n, b, fill):
    out = np.empty(n, dtype=np.float32)
    tb.tb_prep_reference(out.ctypes.data, n, b, fill)
    return out


@pytest.mark.parametrize("n", [1, 15, 16, 17, 383, 384, 1000, 16 * 4096 + 7])
@pytest.mark.parametrize("b", [0, 1, 3, 15])
def test_prep_reference_default_equals_oracle(n, b):
    oracle.assert_equal(_lib_gen(n, b, None), oracle.gen_default(n, b))


def test_prep_reference_default_large_index():
    # indices past 2^24 (the 256 MiB buffers reach 2^26)
    n = (1 << 24) + 1000
    oracle.assert_equal(_lib_gen(n, 1, None), oracle.gen_default(n, 1))


@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 65536 + 3])
@pytest.mark.parametrize("b", [0, 1, 2, 3])
@pytest.mark.parametrize("pct,seed", [(wl.C3_PCT, wl.C3_SEED), ((100, 0, 0, 0, 0), 0),
                                      ((0, 0, 0, 0, 100), 77), ((20, 20, 20, 20, 20), 2**63 + 5)])
def test_prep_reference_compress_equals_oracle(n, b, pct, seed):
    got = _lib_gen(n, b, ("compress", pct, seed))
    oracle.assert_equal(got, oracle.gen_compress(n, b, pct, seed))


def test_prep_reference_compress_c3_buffers_equal_oracle():
    n = 16 << 20
    for b in range(4):
        got = _lib_gen(n, b, ("compress", wl.C3_PCT, wl.C3_SEED))
        oracle.assert_equal(got, oracle.gen_compress(n, b, wl.C3_PCT, wl.C3_SEED))


@pytest.mark.parametrize("n", [1, 2, 3, 10, 1001])
def test_prep_reference_pattern_equals_oracle(n):
    pat = np.array([1.0, -0.0, 3.5e-40, float("inf"), 2.5], dtype=np.float32)
    got = _lib_gen(n, 4, ("pattern", pat))
    oracle.assert_equal(got, oracle.gen_pattern(n, pat))


def test_prep_reference_rejects_bad_config():
    out = np.empty(16, dtype=np.float32)
    with pytest.raises(tb.TBError):
        tb.tb_prep_reference(out.ctypes.data, 16, 0, ("compress", (50, 20, 10, 10, 5), 1))
    with pytest.raises(tb.TBError):
        tb.tb_prep_reference(out.ctypes.data, 16, 0, ("pattern", np.zeros(0, np.float32)))
    with pytest.raises(tb.TBError):
        tb.tb_prep_reference(out.ctypes.data, 16, -1, None)
    with pytest.raises(tb.TBError):
        tb.tb_prep_reference(0, 16, 0, None)


def test_generator_mismatch_is_detected():
    """A single corrupted byte in a library-generated reference is reported."""
    got = _lib_gen(4096, 0, ("compress", wl.C3_PCT, 3))
    got.view(np.uint8)[777] ^= 1
    assert oracle.first_mismatch(got, oracle.gen_compress(4096, 0, wl.C3_PCT, 3)) == 777 // 4


# ---- argument checks of the GPU entry points (rejected before any HIP call) ----

def _st(name, *args):
    return getattr(tb.lib, name)(*args)


def test_reduce_copy_argument_checks():
    srcs = (ctypes.c_void_p * 17)(*([0x1000] * 17))
    assert _st("tb_reduce_copy", 0x1000, srcs, 17, 16, None) == tb.TB_ERR_INVALID        # nsrc > 16
    assert _st("tb_reduce_copy", 0x1000, srcs, -1, 16, None) == tb.TB_ERR_INVALID        # nsrc < 0
    assert _st("tb_reduce_copy", None, srcs, 1, 16, None) == tb.TB_ERR_INVALID           # NULL dst
    assert _st("tb_reduce_copy", 0x1000, None, 2, 16, None) == tb.TB_ERR_INVALID         # NULL srcs
    assert _st("tb_reduce_copy", 0x1002, srcs, 1, 16, None) == tb.TB_ERR_INVALID         # 2-byte aligned dst
    bad = (ctypes.c_void_p * 2)(0x2000, 0x3001)
    assert _st("tb_reduce_copy", 0x1000, bad, 2, 16, None) == tb.TB_ERR_INVALID          # misaligned src
    nul = (ctypes.c_void_p * 2)(0x2000, None)
    assert _st("tb_reduce_copy", 0x1000, nul, 2, 16, None) == tb.TB_ERR_INVALID          # NULL source
    assert _st("tb_reduce_copy", 0x1000, srcs, 1, 2**62, None) == tb.TB_ERR_INVALID      # byte-count overflow
    ovl = (ctypes.c_void_p * 1)(0x1000 + 8)
    assert _st("tb_reduce_copy", 0x1000, ovl, 1, 16, None) == tb.TB_ERR_INVALID          # partial overlap
    assert _st("tb_reduce_copy_ex", 0x1000, srcs, 0, 16, 256, None) == tb.TB_ERR_INVALID  # memset byte > 255
    # zero-length work is a no-op that needs no device
    assert _st("tb_reduce_copy", None, None, 3, 0, None) == tb.TB_OK


def test_batched_copy_argument_checks():
    assert _st("tb_batched_copy", None, 5, None) == tb.TB_ERR_INVALID
    assert _st("tb_batched_copy", 0x1004, 5, None) == tb.TB_ERR_INVALID                  # not 8-byte aligned
    assert _st("tb_batched_copy", None, 0, None) == tb.TB_OK
    assert _st("tb_batched_copy_noalloc", None, 5, None) == tb.TB_ERR_INVALID
    assert _st("tb_batched_copy_noalloc", 0x1004, 5, None) == tb.TB_ERR_INVALID
    assert _st("tb_batched_copy_noalloc", None, 0, None) == tb.TB_OK


def test_timing_hook_needs_no_device():
    assert _st("tb_time_next_launch", None, None) == tb.TB_OK
    assert _st("tb_time_next_launch", 0x1234, None) == tb.TB_OK      # stored only; consumed by a launch
    assert _st("tb_time_next_launch", None, None) == tb.TB_OK        # cleared again


def test_workgroup_cap_needs_no_device():
    for cap in (0, 1, 8, 4096, 2**32 - 1, 0):                        # ends with the default
        assert _st("tb_batched_set_max_workgroups", cap) == tb.TB_OK


def test_batched_mode_hook_checks():
    for bad in (-1, 3, 1 << 20):
        assert _st("tb_batched_set_mode", bad) == tb.TB_ERR_INVALID
    for good in (tb.TB_BC_NO_WAIT, tb.TB_BC_NO_PIECES, tb.TB_BC_NORMAL):   # ends in the default
        assert _st("tb_batched_set_mode", good) == tb.TB_OK


def test_prep_sources_and_gate_argument_checks():
    assert _st("tb_prep_sources", 0x1000, 64, 0, 0x2000, 16, None) == tb.TB_ERR_INVALID    # k == 0
    assert _st("tb_prep_sources", 0x1000, 32, 2, 0x2000, 16, None) == tb.TB_ERR_INVALID    # stride < bytes
    assert _st("tb_prep_sources", None, 64, 2, 0x2000, 16, None) == tb.TB_ERR_INVALID
    assert _st("tb_spin_gate_arm", 0, None) == tb.TB_ERR_INVALID
    assert _st("tb_spin_gate_arm", 60001, None) == tb.TB_ERR_INVALID
    assert _st("tb_spin_gate_release") == tb.TB_ERR_INVALID                                 # never armed


def test_ring_argument_checks():
    out = ctypes.c_void_p(0x1234)
    for nslots, slot_descs, flags in ((0, 8, 0), (1025, 8, 0), (2, 0, 0), (2, (1 << 20) + 1, 0), (2, 8, 2),
                                      (2, 8, 0xFFFFFFFF)):
        assert _st("tb_ring_create", nslots, slot_descs, flags, None, ctypes.byref(out)) == tb.TB_ERR_INVALID
    assert _st("tb_ring_create", 2, 8, tb.TB_RING_STAGED, None, None) == tb.TB_ERR_INVALID   # NULL out
    t, done = ctypes.c_uint64(), ctypes.c_int32()
    assert _st("tb_ring_submit", None, None, 0, ctypes.byref(t)) == tb.TB_ERR_INVALID       # NULL ring
    assert _st("tb_ring_poll", None, 0, ctypes.byref(done)) == tb.TB_ERR_INVALID
    assert _st("tb_ring_wait", None, 0) == tb.TB_ERR_INVALID
    assert _st("tb_ring_destroy", None) == tb.TB_OK                                          # NULL: no-op


def test_product_package_does_not_use_oracle():
    """The HIP package and the oracle share nothing and never import each other."""
    pkg = os.path.join(ROOT, "copy_reduce_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
    text = open(os.path.join(ROOT, "oracle", "oracle.c")).read() + open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert "copy_reduce_amd" not in text.replace("(copy_reduce_amd/)", "") and "tb.h" not in text


def test_c_consumer_calls_every_entry_point():
    """tests/capi/capi_check.c (run on the GPU by test_gpu_capi.py) calls every
    entry point include/tb.h declares, so the whole boundary is exercised once
    from plain C without the Python binding."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    header = open(os.path.join(root, "include", "tb.h")).read()
    consumer = open(os.path.join(root, "tests", "capi", "capi_check.c")).read()
    declared = sorted(set(re.findall(r"^(?:int|const char \*)\s*(tb_\w+)\s*\(", header, re.M)))
    assert declared
    assert [d for d in declared if d + "(" not in consumer] == []
