"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the oracle and of
libtb's host half (slice geometry, rotation, the PrepareReference
generators, argument checks), each driven over small and edge-case sizes by a
C/C++ driver under tests/sanitize/.  Built with gcc/g++ (host code only; the
library's kernel object is linked in unsanitised).  No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-D_POSIX_C_SOURCE=199309L"] + SAN +
         ["-o", exe, "oracle/oracle.c", "tests/sanitize/oracle_driver.c"])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1"))
    assert "oracle sanitizer run ok" in r.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("HIP headers are not installed")
    kobj = os.path.join(ROOT, "copy_reduce_amd", "_build", "tb_kernels.o")
    if not os.path.exists(kobj):   # the kernels, unsanitised, for the symbols the host code launches
        kobj = str(tmp_path / "tb_kernels.o")
        _run([shutil.which("hipcc") or "/opt/rocm/bin/hipcc", "-std=c++17", "-O3", "-fPIC", "-x", "hip",
              "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Iinclude", "-Icopy_reduce_amd/csrc", "-c", "copy_reduce_amd/csrc/tb_kernels.hip", "-o", kobj])
    common = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-Iinclude", "-Icopy_reduce_amd/csrc"] + SAN
    objs = []
    for src in ("copy_reduce_amd/csrc/tb_host.cpp", "copy_reduce_amd/csrc/tb_gen.cpp", "copy_reduce_amd/csrc/tb_ring.cpp",
                "tests/sanitize/host_driver.cpp"):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++"] + common + ["-c", src, "-o", o])
        objs.append(o)
    exe = str(tmp_path / "host_san")
    _run(["g++", "-fsanitize=address,undefined", "-o", exe] + objs +
         [kobj, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    # the HIP runtime keeps allocations for the life of the process: no leak report
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1"))
    assert "host sanitizer run ok" in r.stdout
