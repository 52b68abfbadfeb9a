"""Build the CPU oracle (oracle/liboracle.so) with plain gcc.

Test infrastructure only: see oracle/oracle.c.  The flags keep binary32
arithmetic exactly as written: x86-64 SSE scalar floats, no fast-math, no
floating-point contraction, no vectorisation that could reorder anything.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-std=c11", "-O2", "-fPIC", "-shared",
    "-fno-fast-math", "-ffp-contract=off", "-fno-tree-vectorize",
    "-mfpmath=sse", "-msse2",
    "-Wall", "-Wextra", "-Werror",
]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
