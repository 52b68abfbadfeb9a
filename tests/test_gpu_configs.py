"""Parity at the benchmark configurations' full sizes, in the launch
configuration the benchmark times (rotated pointers, same entry points):
C1 4 MiB copy K=64 (validated after every iteration, ALWAYS_VALIDATE=1),
C2 two-source 256 MiB rotation on and R=0, C3 four-source 64 MiB fillCompress
K=4, the C5 copy sweep 8-512 MiB, C4 47,520 scattered copies and the C5 mixed
KV batch (whole 4 GiB pool compared)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu


def _reduce_config(torch, w: wl.ReduceWorkload, always_validate: bool):
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import RotatedSources
    rs = RotatedSources(w.nsrc, w.nfloats, w.rotate_bytes, fill=w.fill)
    assert rs.k == oracle.num_slices(w.num_bytes, w.rotate_bytes)
    exp = oracle.ref_reduce([oracle.gen_source(w.nfloats, b, w.fill) for b in range(w.nsrc)])
    dst = torch.zeros(w.nfloats, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(-w.warmup, w.iters):
        tb.tb_reduce_copy(int(dst.data_ptr()), rs.pointers(i), w.nfloats, stream)
        if always_validate and i >= 0:
            torch.cuda.synchronize()
            oracle.assert_equal(dst.cpu().numpy(), exp, f"iteration {i}")
    torch.cuda.synchronize()
    oracle.assert_equal(dst.cpu().numpy(), exp)


@pytest.mark.parametrize("name,always", [("c1_copy_4MiB_rot", True), ("c2_reduce2_256MiB_rot", False),
                                         ("c2_reduce2_256MiB_norot", False), ("c3_reduce4_64MiB_compress", True)])
def test_reduce_configs_full_size(name, always):
    torch = require_gpu()
    w = wl.REDUCE_CONFIGS[name]
    note(f"config {name} nsrc={w.nsrc} nfloats={w.nfloats} R={w.rotate_bytes}")
    _reduce_config(torch, w, always)


@pytest.mark.parametrize("nbytes", wl.SWEEP_BYTES)
@pytest.mark.parametrize("rotate", [True, False])
def test_copy_sweep_full_size(nbytes, rotate):
    torch = require_gpu()
    w = wl.sweep_workload(nbytes, rotate)
    note(f"sweep {w.name}")
    _reduce_config(torch, w, False)


def _batch_config(torch, batch: wl.Batch, replicas: int):
    """Source image replicated `replicas` times; launch i uses replica i mod K_b
    (the rotation rule applied to the batch's sources)."""
    import copy_reduce_amd as tb
    from copy_reduce_amd.torch_api import make_desc
    stride = tb.tb_slice_stride(batch.src_bytes)
    src = torch.empty(replicas * stride, dtype=torch.uint8, device="cuda")
    host = torch.from_numpy(batch.payload)
    for r in range(replicas):
        src[r * stride:r * stride + batch.src_bytes].copy_(host)
    pool = torch.full((batch.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    descs = [make_desc(batch.desc, int(src.data_ptr()) + r * stride, int(pool.data_ptr())) for r in range(replicas)]
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(-3, 10):
        r = oracle.slice_of(i, replicas)
        tb.tb_batched_copy(int(descs[r].data_ptr()), batch.ncopies, stream)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    del pool, src
    exp = np.full(batch.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    oracle.ref_batch(exp, batch.payload, batch.desc)
    oracle.assert_equal(got, exp)


@pytest.mark.parametrize("which", ["c4", "c5"])
def test_batched_configs_full_size(which):
    torch = require_gpu()
    batch = wl.batch_c4() if which == "c4" else wl.batch_c5()
    import copy_reduce_amd as tb
    replicas = tb.tb_num_slices(batch.total_bytes, wl.DEFAULT_ROTATE_BYTES)
    note(f"config {batch.name} ncopies={batch.ncopies} bytes={batch.total_bytes} replicas={replicas}")
    _batch_config(torch, batch, replicas)
