"""The copy baselines bench.py times beside the kernels: the HIP runtime's own
device-to-device copy (with a kernel, and with a copy engine) and one
hipMemcpyAsync per descriptor.  These check that the harness drives them on the
right addresses: their bytes must equal the oracle's."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

KINDS = ["HIP_MEMCPY_D2D", "HIP_MEMCPY_D2D_NOCU"]


@pytest.mark.parametrize("kind", KINDS)
def test_runtime_copy_of_rotated_slices(kind):
    torch = require_gpu()
    import bench
    from copy_reduce_amd.torch_api import RotatedSources
    memcpy = bench.hip_memcpy_fn()
    n = (1 << 18) + 3
    rs = RotatedSources(1, n, 4 * n * 4)
    assert rs.k == 4
    dst = torch.full((n,), -1.0, dtype=torch.float32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    note(f"baseline runtime copy kind={kind} n={n}")
    for i in range(-3, 10):
        (p,) = rs.pointers(i)
        assert memcpy(int(dst.data_ptr()), p, n * 4, getattr(bench, kind), sh) == 0
    torch.cuda.synchronize()
    oracle.assert_equal(dst.cpu().numpy(), oracle.gen_source(n, 0, None))


@pytest.mark.parametrize("kind", KINDS)
def test_one_call_per_descriptor(kind):
    torch = require_gpu()
    import bench
    memcpy = bench.hip_memcpy_fn()
    b = wl.batch_random(21, 400, max_bytes=20000, pool_bytes=16 << 20)
    src = torch.from_numpy(b.payload).to("cuda")
    pool = torch.full((b.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    d = b.desc.astype(np.int64)
    srcs = (d[:, 0] + int(src.data_ptr())).tolist()
    dsts = (d[:, 1] + int(pool.data_ptr())).tolist()
    note(f"baseline per-descriptor kind={kind} n={b.ncopies}")
    _, rc = bench.percopy_submit(memcpy, srcs, dsts, d[:, 2].tolist(), getattr(bench, kind),
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    exp = np.full(b.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    oracle.ref_batch(exp, b.payload, b.desc)
    oracle.assert_equal(pool.cpu().numpy(), exp)
    assert bench.oracle_pool_ok([pool], b)
    k = int(np.flatnonzero(b.desc[:, 2] > 0)[0])
    pool[int(b.desc[k, 1])] ^= 0xFF        # one flipped byte must be caught
    assert not bench.oracle_pool_ok([pool], b)
