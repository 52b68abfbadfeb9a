"""The C ABI used from a plain C11 program (tests/capi/capi_check.c): device
memory from the HIP runtime's C API, libtb.so called directly, no Python
binding and no torch in the process; every entry point tb.h declares is
called.  A consumer-side check of the boundary; parity against the oracle is
tested elsewhere."""
import os
import subprocess

import pytest

from gpu_util import note

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "capi", "capi_check")

pytestmark = pytest.mark.gpu


def test_c_program_uses_the_abi():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: build first (python -c 'import __graft_entry__ as g; g.build()')")
    note("C-ABI consumer: every entry point of tb.h from plain C (reduce-copy incl. the LDS path, slices and "
         "rotation, gate and timing, batched copy, no-alloc copy, both ring kinds, argument checks)")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout}\n{r.stderr}"
    assert "capi ok" in r.stdout
