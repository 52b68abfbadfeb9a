"""Build libtb.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

Every HIP translation unit is compiled for gfx950 only, without fast-math
(the reduce-copy's fixed addition order is part of its contract) and with
packed fp32 instructions disabled.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtb.so")
ARCH = "gfx950"

SOURCES = ["tb_host.cpp", "tb_gen.cpp", "tb_ring.cpp", "tb_kernels.hip"]
# The measuring instruments of bench.py --roofs: a library of their own.
ROOFS_SOURCES = ["tb_roofs.hip"]
ROOFS_LIB = os.path.join(PKG, "libtb_roofs.so")

COMMON = [
    "-std=c++17", "-O3", "-fPIC", "-Wall", "-Wextra", "-Werror",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
DEVICE = [
    "-x", "hip", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libtb needs the ROCm toolchain to build")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link copy_reduce_amd/libtb.so and
    copy_reduce_amd/libtb_roofs.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + ROOFS_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in ROOFS_SOURCES], ROOFS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
