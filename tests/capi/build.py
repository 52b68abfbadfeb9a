"""Build tests/capi/capi_check: the C-ABI consumer check, plain C11 (gcc),
linked against copy_reduce_amd/libtb.so and the HIP runtime."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
OUT = os.path.join(HERE, "capi_check")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "capi_check.c"), "-o", OUT + ".tmp",
           "-L", os.path.join(ROOT, "copy_reduce_amd"), "-ltb", "-Wl,-rpath,$ORIGIN/../../copy_reduce_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C-ABI check failed to build:\n{r.stdout}\n{r.stderr}")
    os.replace(OUT + ".tmp", OUT)
    return OUT
