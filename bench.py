#!/usr/bin/env python3
"""Benchmark of the transfer hot path on one MI355X (gfx950).

One step = one pass of the whole hot path over one batch of synthetic input:
  1. source-slice rotation (host arithmetic, tb_rotate_sources),
  2. the two-source fp32 reduce-copy over 256 MiB buffers (tb_reduce_copy),
  3. the 47,520-copy batched scattered copy into a 4 GiB pool (tb_batched_copy),
all enqueued on one stream.  Inputs are prepared (and resident in HBM) before
the timed region; K steps are enqueued behind the spin gate between two HIP
events (the value), then enqueued again with every launch carrying its own
start and stop event (per-kernel times, on the stream each launch runs on).

Default output is ONE JSON line:
  value        whole-step throughput, algorithmic HBM GB/s (decimal):
               (N+1) x numBytes for the reduce-copy + 2 x sum(bytes) for the batch
  roofline     the dominant kernel (the reduce-copy) against 8 TB/s HBM
  cpu_baseline the oracle timed on one host core over the same step
--suite additionally prints one line per configuration (C1-C5, sweep);
--cpu-suite times the oracle alone on one host core for every configuration.
The other flags (--baselines, --cache-study, --roofs, --interference, --ring,
--scatter-study, --misaligned, --calibrate-copy) each run one study instead; see --help.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HBM GB/s & % of peak (rotated reduce-copy); GB/s + copies/s (batched scatter)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
GATE_TIMEOUT_MS = 20000
DST_ROTATE_BYTES = 1 << 30      # the bench step's reduce-copy destination rotates over this many bytes
BATCH_DST_ROTATE_BYTES = 512 << 20   # and the batched copy's destination pools over this many payload bytes
CPU_BUDGET_S = 10.0             # single-core work of the cpu_baseline leg


def _sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only
    if it was taken on the kernels as they are now (same source hash)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "copy_reduce_amd", "csrc", "tb_kernels.hip")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != _sha256(src):
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


class Timed:
    """Enqueue a sequence of launches behind the spin gate with an event at
    every boundary; per-launch milliseconds come from consecutive events."""

    def __init__(self, torch, tb, stream):
        self.torch, self.tb, self.stream = torch, tb, stream

    def run(self, launches):
        torch, tb, s = self.torch, self.tb, self.stream
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tb.tb_spin_gate_arm(GATE_TIMEOUT_MS, s.cuda_stream)
        evs[0].record(s)
        for j, fn in enumerate(launches):
            fn()
            evs[j + 1].record(s)
        tb.tb_spin_gate_release()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if tb.tb_spin_gate_status() != tb.TB_OK:
            raise RuntimeError("spin gate timed out: the timed launches were not gated")
        ms = [evs[j].elapsed_time(evs[j + 1]) for j in range(len(launches))]
        return ms, evs[0].elapsed_time(evs[-1]), wall


def run_whole(torch, tb, stream, launches):
    """The launches behind the spin gate with one event before the first and
    one after the last (nvbandwidth's protocol): (ms, wall seconds)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tb.tb_spin_gate_arm(GATE_TIMEOUT_MS, stream.cuda_stream)
    e0.record(stream)
    for fn in launches:
        fn()
    e1.record(stream)
    tb.tb_spin_gate_release()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if tb.tb_spin_gate_status() != tb.TB_OK:
        raise RuntimeError("spin gate timed out: the timed launches were not gated")
    return e0.elapsed_time(e1), wall


def run_launch_events(torch, tb, stream, launches):
    """The launches behind the spin gate, each carrying its own start and stop
    event (tb_time_next_launch), so no event command sits between kernels:
    (per-launch ms, ms from the first start to the last stop)."""
    def made():
        evs = [torch.cuda.Event(enable_timing=True) for _ in launches]
        for e in evs:                  # a first record creates the underlying event
            e.record(stream)
        return evs
    st, sp = made(), made()
    torch.cuda.synchronize()
    tb.tb_spin_gate_arm(GATE_TIMEOUT_MS, stream.cuda_stream)
    for j, fn in enumerate(launches):
        tb.tb_time_next_launch(st[j].cuda_event, sp[j].cuda_event)
        fn()
    tb.tb_spin_gate_release()
    torch.cuda.synchronize()
    if tb.tb_spin_gate_status() != tb.TB_OK:
        raise RuntimeError("spin gate timed out: the timed launches were not gated")
    return [st[j].elapsed_time(sp[j]) for j in range(len(launches))], st[0].elapsed_time(sp[-1])


def device_record(torch, tb):
    """Name, CU count and the partition modes the measurement ran under (the
    cache behaviour rotation guards against depends on them)."""
    import glob
    props = torch.cuda.get_device_properties(0)
    rec = {"name": props.name or torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
           "hip_runtime": getattr(torch.version, "hip", None),
           "cu_count": tb.tb_launch_info()["cu_count"],
           "hbm_bytes": int(props.total_memory)}
    for key, fname in (("compute_partition", "current_compute_partition"),
                       ("memory_partition", "current_memory_partition")):
        vals = set()
        for path in glob.glob(f"/sys/class/drm/card*/device/{fname}"):
            try:
                with open(path) as f:
                    vals.add(f.read().strip())
            except OSError:
                pass
        rec[key] = "/".join(sorted(vals)) if vals else "unknown"
    return rec


# ---------------------------------------------------------------------------
# workload set-up (untimed)
# ---------------------------------------------------------------------------

def setup_reduce(torch, w):
    from copy_reduce_amd.torch_api import RotatedSources
    rs = RotatedSources(w.nsrc, w.nfloats, w.rotate_bytes, fill=w.fill)
    dst = torch.zeros(max(1, w.nfloats), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    return rs, dst


def setup_batch(torch, tb, batch, rotate_bytes, dst_rotate_bytes=0):
    """K_b source replicas (the slice-count rule over the batch's source bytes)
    and K_p destination pools (the same rule over dst_rotate_bytes; one pool
    when it is 0), each pool pre-filled with 0xA5; one descriptor array per
    (replica, pool).  Iteration i reads replica i mod K_b and writes pool
    i mod K_p."""
    import workloads as wl
    from copy_reduce_amd.torch_api import make_desc
    batch.check()
    kb = tb.tb_num_slices(batch.total_bytes, rotate_bytes)
    kp = tb.tb_num_slices(batch.total_bytes, dst_rotate_bytes)
    stride = tb.tb_slice_stride(batch.src_bytes)
    pstride = tb.tb_slice_stride(batch.pool_bytes)
    src = torch.empty(max(1, kb * stride), dtype=torch.uint8, device="cuda")
    host = torch.from_numpy(batch.payload).pin_memory()
    for r in range(kb):
        src[r * stride:r * stride + batch.src_bytes].copy_(host, non_blocking=True)
    pools = torch.full((kp * pstride,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    base, pbase = int(src.data_ptr()), int(pools.data_ptr())
    descs = {(base + r * stride, pbase + p * pstride): make_desc(batch.desc, base + r * stride, pbase + p * pstride)
             for r in range(kb) for p in range(kp)}
    torch.cuda.synchronize()
    return {"kb": kb, "stride": stride, "src": src, "descs": descs, "base": base,
            "kp": kp, "pstride": pstride, "pools": pools, "pbase": pbase,
            "pool_views": [pools[p * pstride:p * pstride + batch.pool_bytes] for p in range(kp)],
            "pool": pools[:batch.pool_bytes]}


def replica_of(tb, b, i):
    """Source replica iteration i reads, (i mod K_b), via the library's rotation."""
    (addr,) = tb.tb_rotate_sources([b["base"]], b["stride"], b["kb"], i)
    return (addr - b["base"]) // b["stride"]


def batch_desc_for(tb, b, i):
    """Descriptor array of iteration i: source replica and destination pool by
    the library's rotation (slice i mod K)."""
    (src,) = tb.tb_rotate_sources([b["base"]], b["stride"], b["kb"], i)
    (pool,) = tb.tb_rotate_sources([b["pbase"]], b["pstride"], b["kp"], i)
    return b["descs"][(src, pool)]


def pools_written(b, first, last):
    """The destination pools iterations first .. last - 1 wrote."""
    kp = b["kp"]
    return [b["pool_views"][p] for p in sorted({(i % kp + kp) % kp for i in range(first, last)})]


# ---------------------------------------------------------------------------
# the benchmark step
# ---------------------------------------------------------------------------

def main_line(args, torch, tb, wl):
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    w = wl.REDUCE_CONFIGS["c2_reduce2_256MiB_rot"]
    rs, dst = setup_reduce(torch, w)
    batch = wl.batch_c4()
    b = setup_batch(torch, tb, batch, wl.DEFAULT_ROTATE_BYTES, BATCH_DST_ROTATE_BYTES)
    # The destination rotates too, by the slice rule over DST_ROTATE_BYTES: at
    # 256 MiB per buffer the source rule gives K = 1, and a fixed 256 MiB
    # destination written with stores that allocate in the 256 MB memory-side
    # cache stays there and has its rewrites absorbed; over K_d slices every
    # launch writes lines no recent launch wrote, so the timed rate is the HBM
    # rate whatever the store policy (the library's stores do not allocate
    # there, and the fixed-destination pass beside it reads the same).
    kd = tb.tb_num_slices(rs.num_bytes, DST_ROTATE_BYTES)
    dsts = torch.zeros(kd * rs.stride // 4, dtype=torch.float32, device="cuda")
    dst_base = int(dsts.data_ptr())
    dst_fixed = int(dst.data_ptr())

    def dst_for(i):
        return tb.tb_rotate_sources([dst_base], rs.stride, kd, i)[0]

    def rc(i, fixed=False):
        ptrs = rs.pointers(i)                      # rotation: before the launch, untimed work
        d = dst_fixed if fixed else dst_for(i)
        return lambda: tb.tb_reduce_copy(d, ptrs, w.nfloats, sh)

    def bc(i):
        d = batch_desc_for(tb, b, i)
        return lambda: tb.tb_batched_copy(int(d.data_ptr()), batch.ncopies, sh)

    for i in range(-args.warmup, 0):
        rc(i)()
        bc(i)()
    torch.cuda.synchronize()

    launches = []
    for i in range(args.steps):
        launches += [rc(i), bc(i)]
    # the K steps as one timed region (the value), then the same K steps again
    # with each launch carrying its own events (the per-kernel figures)
    total_ms, wall = run_whole(torch, tb, stream, launches)
    ms, total_ms_launch_events = run_launch_events(torch, tb, stream, launches)
    rc_ms, bc_ms = ms[0::2], ms[1::2]
    # the pages' literal protocol beside it: the same steps with one fixed destination
    for i in range(-args.warmup, 0):
        rc(i, fixed=True)()
        bc(i)()
    fixed = []
    for i in range(args.steps):
        fixed += [rc(i, fixed=True), bc(i)]
    ms_fixed, _ = run_launch_events(torch, tb, stream, fixed)
    rc_fixed_ms = ms_fixed[0::2]

    rc_bytes, bc_bytes = w.algorithmic_bytes, batch.algorithmic_bytes
    step_bytes = rc_bytes + bc_bytes
    value = args.steps * step_bytes / (total_ms * 1e-3) / 1e9
    rc_mean, bc_mean = statistics.mean(rc_ms), statistics.mean(bc_ms)
    rc_gbps = rc_bytes / (rc_mean * 1e-3) / 1e9
    bc_gbps = bc_bytes / (bc_mean * 1e-3) / 1e9
    info = tb.tb_launch_info(w.nfloats, w.nsrc, batch.ncopies)
    traffic = _traffic("reduce_copy")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "rotated 2-source fp32 reduce-copy, 256 MiB per buffer (67,108,864 floats, "
                        "PrepSrcValue sources, SRC_ROTATE_BYTES=256 MiB -> K=1; destination rotated over "
                        f"K_d={kd} slices, 1 GiB) + batched scattered copy "
                        "of 47,520 copies log-uniform 64 B-16 KiB into random 16 KiB slots of a 4 GiB pool "
                        f"(K_b={b['kb']} source replicas, K_p={b['kp']} destination pools), one of each per step",
            "reduce_copy": {"nsrc": w.nsrc, "nfloats": w.nfloats, "rotate_bytes": w.rotate_bytes, "k": rs.k,
                            "dst_rotate_bytes": DST_ROTATE_BYTES, "k_dst": kd, "bytes_per_launch": rc_bytes},
            "batched_copy": {"ncopies": batch.ncopies, "payload_bytes": batch.total_bytes,
                             "bytes_per_launch": bc_bytes, "replicas": b["kb"], "dst_rotate_bytes":
                             BATCH_DST_ROTATE_BYTES, "pools": b["kp"]},
            "launch": info,
        },
        "device": device_record(torch, tb),
        "parts": {
            "reduce_copy": {"ms_mean": round(rc_mean, 5), "ms_min": round(min(rc_ms), 5),
                            "ms_max": round(max(rc_ms), 5), "gbps": round(rc_gbps, 1),
                            "frac_of_peak": round(rc_gbps / HBM_PEAK_GBPS, 4),
                            "fixed_dst": {
                                "note": "the same steps with one fixed destination, as the pages time it; the "
                                        "reduce-copy's stores do not allocate in the 256 MB memory-side cache, so "
                                        "a rewritten destination is not served from it and this too is an HBM rate",
                                "ms_mean": round(statistics.mean(rc_fixed_ms), 5),
                                "frac_of_peak": round(rc_bytes / (statistics.mean(rc_fixed_ms) * 1e-3) / 1e9
                                                      / HBM_PEAK_GBPS, 4)}},
            "batched_copy": {"ms_mean": round(bc_mean, 5), "ms_min": round(min(bc_ms), 5),
                             "ms_max": round(max(bc_ms), 5), "gbps": round(bc_gbps, 1),
                             "frac_of_peak": round(bc_gbps / HBM_PEAK_GBPS, 4),
                             "copies_per_s": round(batch.ncopies / (bc_mean * 1e-3), 1)},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "reduce_copy",
            "achieved": round(rc_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(rc_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "wall_s_timed_region": round(wall, 4),
        "timing": {
            "value": "HIP events before the first and after the last of the K timed steps, behind a spin "
                     "kernel (nvbandwidth's protocol)",
            "parts_and_roofline": "the same K steps again, each launch carrying its own start and stop event "
                                  "(hipExtLaunchKernel launch events), on the launch stream",
            "ms_per_step_with_launch_events": round(total_ms_launch_events / args.steps, 4),
        },
    }

    if not args.no_cpu_baseline:
        written = sorted({(i % kd + kd) % kd for i in range(-args.warmup, args.steps)})
        views = [dsts[s * rs.stride // 4:s * rs.stride // 4 + w.nfloats] for s in written] + [dst]
        line["cpu_baseline"], line["validated"] = cpu_baseline(torch, w, batch, views,
                                                               pools_written(b, -args.warmup, args.steps))
    print(json.dumps(line), flush=True)
    return line


# ---------------------------------------------------------------------------
# The oracle leg: the CPU oracle timed as the baseline, and the checks of the
# GPU results against it.  These functions are the only place bench.py uses
# oracle/ (the transfer path never does).
# ---------------------------------------------------------------------------

def cpu_baseline(torch, w, batch, dsts, pools):
    """The oracle, as it stands, timed on one host core over the full step,
    repeated for about CPU_BUDGET_S seconds (median); also checks the GPU
    results of the timed run against it: every destination slice the
    reduce-copy wrote, and the whole pool."""
    import numpy as np

    import oracle
    import workloads as wl
    srcs = [oracle.gen_source(w.nfloats, b, w.fill) for b in range(w.nsrc)]
    image = np.full(batch.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    # whole steps, repeated until about 10 s of single-core work (at least 3, at most 400)
    t_rc, t_bc, exp = [], [], None
    while len(t_rc) < 3 or (sum(t_rc) + sum(t_bc) < CPU_BUDGET_S and len(t_rc) < 400):
        t, exp = oracle.time_ref_reduce(srcs)
        t_rc.append(t)
        t_bc.append(oracle.time_ref_batch(image, batch.payload, batch.desc))
    rc_s, bc_s = statistics.median(t_rc), statistics.median(t_bc)
    step_bytes = w.algorithmic_bytes + batch.algorithmic_bytes
    validated = {
        "reduce_copy": all(oracle.first_mismatch(d.cpu().numpy(), exp) == -1 for d in dsts),
        "batched_copy": all(oracle.first_mismatch(p.cpu().numpy(), image) == -1 for p in pools),
    }
    cpu = {
        "value": round(step_bytes / (rc_s + bc_s) / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the full step on one core, repeated {len(t_rc)} times ({sum(t_rc) + sum(t_bc):.1f} s of work), "
                  "median: the 2-source fp32 reduce over 67,108,864 floats and the 47,520 descriptor memcpys "
                  "into a 4 GiB host pool image",
        "steps_timed": len(t_rc),
        "reduce_copy_gbps": round(w.algorithmic_bytes / rc_s / 1e9, 3),
        "batched_copy_gbps": round(batch.algorithmic_bytes / bc_s / 1e9, 3),
        "batched_copies_per_s": round(batch.ncopies / bc_s, 1),
        "host_cores_total": os.cpu_count(),
        "cpu_model": _cpu_model(),
    }
    return cpu, validated


def oracle_reduce_ok(dsts, w=None, srcs=None):
    """Every element of each device view in dsts against the oracle's
    fixed-order sum: of the workload's sources (oracle.gen_source) when w is
    given, else of the device source views srcs, read back."""
    import oracle
    if w is not None:
        host = [oracle.gen_source(w.nfloats, b, w.fill) for b in range(w.nsrc)]
    else:
        host = [x.cpu().numpy() for x in srcs]
    exp = oracle.ref_reduce(host)
    return all(oracle.first_mismatch(d.cpu().numpy(), exp) == -1 for d in dsts)


def oracle_pool_ok(pools, batch, src_shift=0):
    """Every byte of each pool (device uint8 views of at least batch.pool_bytes)
    against the oracle's per-descriptor memcpy of the batch into an image
    pre-filled with 0xA5.  src_shift: every descriptor read src_shift bytes
    past its source offset, in the batch's source image followed by zero
    bytes (as the misaligned study lays it out)."""
    import numpy as np

    import oracle
    import workloads as wl
    exp = np.full(batch.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
    image = np.zeros(batch.src_bytes + src_shift, dtype=np.uint8)
    image[:batch.src_bytes] = batch.payload[:batch.src_bytes]
    d = batch.desc.astype(np.uint64).copy()
    d[:, 0] += np.uint64(src_shift)
    oracle.ref_batch(exp, image, d)
    return all(oracle.first_mismatch(p[:batch.pool_bytes].cpu().numpy(), exp) == -1 for p in pools)


def cpu_baseline_suite(args, wl):
    """The cpu_baseline leg for every configuration: the oracle, as it stands,
    timed on one host core (median of 3) -- the cumulative reduce over nfloats
    for C1-C3 and the sweep (rotation does not change the host computation),
    the per-descriptor memcpy into a 4 GiB host pool image for C4 and C5a.
    One JSON line per configuration; no GPU work."""
    import numpy as np

    import oracle
    common = {"cores": 1, "kind": "oracle", "host_cores_total": os.cpu_count(), "cpu_model": _cpu_model()}
    works = [wl.REDUCE_CONFIGS[k] for k in ("c1_copy_4MiB_rot", "c2_reduce2_256MiB_rot", "c3_reduce4_64MiB_compress")]
    works += [wl.sweep_workload(nb, True) for nb in wl.SWEEP_BYTES]
    for w in works:
        srcs = [oracle.gen_source(w.nfloats, b, w.fill) for b in range(w.nsrc)]
        secs = statistics.median([oracle.time_ref_reduce(srcs)[0] for _ in range(3)])
        rec = {"config": w.name, "nsrc": w.nsrc,
               "nfloats": w.nfloats, "seconds": round(secs, 6),
               "gbps": round(w.algorithmic_bytes / secs / 1e9, 3), **common}
        print(json.dumps({"cpu_suite": rec}), flush=True)
        del srcs
    for batch in (wl.batch_c4(), wl.batch_c5()):
        image = np.full(batch.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
        secs = statistics.median([oracle.time_ref_batch(image, batch.payload, batch.desc) for _ in range(3)])
        rec = {"config": batch.name, "ncopies": batch.ncopies, "seconds": round(secs, 6),
               "gbps": round(batch.algorithmic_bytes / secs / 1e9, 3),
               "copies_per_s": round(batch.ncopies / secs, 1), **common}
        print(json.dumps({"cpu_suite": rec}), flush=True)
        del image


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
# --suite: every configuration, one JSON line each
# ---------------------------------------------------------------------------

def _kernel_and_loop(nbytes, kernel_ms, whole_ms, steps):
    """Two more readings of the same launches: each kernel's own duration
    (launch-carried events) and the loop's rate with events at its two ends."""
    kg = nbytes / (kernel_ms * 1e-3) / 1e9
    lg = steps * nbytes / (whole_ms * 1e-3) / 1e9
    return {"ms_kernel": round(kernel_ms, 5), "kernel_frac_of_peak": round(kg / HBM_PEAK_GBPS, 4),
            "loop_ms_per_launch": round(whole_ms / steps, 5), "loop_frac_of_peak": round(lg / HBM_PEAK_GBPS, 4)}


def suite(args, torch, tb, wl):
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    timer = Timed(torch, tb, stream)

    def reduce_line(w, reps=1, rotate_dst=False):
        """rotate_dst: also rotate the destination over K slices (same rule as the
        sources).  Not the pages' method (they rotate sources only); it shows
        the rate with a destination that is not resident in the memory-side cache."""
        rs, dst = setup_reduce(torch, w)
        kd = rs.k if rotate_dst else 1
        dsts = torch.empty(max(1, kd * rs.stride), dtype=torch.uint8, device="cuda") if rotate_dst else None
        dbase = int(dsts.data_ptr()) if rotate_dst else int(dst.data_ptr())

        def dptr_for(i):
            if not rotate_dst:
                return dbase
            return tb.tb_rotate_sources([dbase], rs.stride, kd, i)[0]

        # cold: the first launch after prep, timed on its own (a diagnostic;
        # the figure is the warm mean below)
        i0 = -args.warmup if args.warmup else 0
        cold_ms, _, _ = timer.run([lambda p=rs.pointers(i0), dp=dptr_for(i0): tb.tb_reduce_copy(dp, p, w.nfloats, sh)])
        means = []
        for rep in range(reps):
            for i in range(-args.warmup + (1 if rep == 0 and args.warmup else 0), 0):
                tb.tb_reduce_copy(dptr_for(i), rs.pointers(i), w.nfloats, sh)
            launches = []
            for i in range(args.steps):
                ptrs, dp = rs.pointers(i), dptr_for(i)
                launches.append(lambda p=ptrs, dp=dp: tb.tb_reduce_copy(dp, p, w.nfloats, sh))
            ms, total, _ = timer.run(launches)
            kms, _ = run_launch_events(torch, tb, stream, launches)
            whole, _ = run_whole(torch, tb, stream, launches)
            means.append((statistics.mean(ms), min(ms), max(ms), total, statistics.mean(kms), whole))
        med = sorted(means)[len(means) // 2]
        gbps = w.algorithmic_bytes / (med[0] * 1e-3) / 1e9
        out = {"config": w.name + ("_dstrot" if rotate_dst else ""), "nsrc": w.nsrc, "nfloats": w.nfloats,
               "k": rs.k, "reps": reps,
               "ms_mean": round(med[0], 5), "ms_min": round(med[1], 5), "ms_max": round(med[2], 5),
               "ms_cold": round(cold_ms[0], 5),
               "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
               "aggregate_gbps": round(args.steps * w.algorithmic_bytes / (med[3] * 1e-3) / 1e9, 1)}
        out.update(_kernel_and_loop(w.algorithmic_bytes, med[4], med[5], args.steps))
        del rs, dst, dsts
        torch.cuda.empty_cache()
        return out

    def batch_line(batch, rotate_bytes, tag, dst_rotate_bytes=0):
        """dst_rotate_bytes: rotate the destination pool too (K_p pools by the
        slice rule), so no launch rewrites lines a recent launch left in the
        memory-side cache; not the pages' method (they rotate sources only)."""
        b = setup_batch(torch, tb, batch, rotate_bytes, dst_rotate_bytes)
        # The library creates a stream's scratch on its first call there: one
        # descriptor of zero bytes before the cold launch keeps that allocation
        # out of the cold figure (the kernel copies nothing for it).
        none = torch.tensor([[b["base"], int(b["pool"].data_ptr()), 0]], dtype=torch.int64, device="cuda")
        tb.tb_batched_copy(int(none.data_ptr()), 1, sh)
        torch.cuda.synchronize()
        i0 = -args.warmup if args.warmup else 0
        d0 = batch_desc_for(tb, b, i0)
        cold_ms, _, _ = timer.run([lambda: tb.tb_batched_copy(int(d0.data_ptr()), batch.ncopies, sh)])
        for i in range(-args.warmup + (1 if args.warmup else 0), 0):
            d = batch_desc_for(tb, b, i)
            tb.tb_batched_copy(int(d.data_ptr()), batch.ncopies, sh)
        launches = []
        for i in range(args.steps):
            d = batch_desc_for(tb, b, i)
            launches.append(lambda d=d: tb.tb_batched_copy(int(d.data_ptr()), batch.ncopies, sh))
        ms, total, _ = timer.run(launches)
        kms, _ = run_launch_events(torch, tb, stream, launches)
        whole, _ = run_whole(torch, tb, stream, launches)
        mean = statistics.mean(ms)
        gbps = batch.algorithmic_bytes / (mean * 1e-3) / 1e9
        out = {"config": f"{batch.name}_{tag}", "ncopies": batch.ncopies, "payload_bytes": batch.total_bytes,
               "replicas": b["kb"], "pools": b["kp"], "ms_mean": round(mean, 5), "ms_min": round(min(ms), 5),
               "ms_max": round(max(ms), 5), "ms_cold": round(cold_ms[0], 5), "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
               "copies_per_s": round(batch.ncopies / (mean * 1e-3), 1)}
        out.update(_kernel_and_loop(batch.algorithmic_bytes, statistics.mean(kms), whole, args.steps))
        del b
        torch.cuda.empty_cache()
        return out

    # controls beyond the pages' method: destination rotated too (R = 1 GiB for C2 so that K > 1)
    c2cold = wl.ReduceWorkload("c2_reduce2_256MiB_R1GiB", 2, 64 << 20, 4 * wl.DEFAULT_ROTATE_BYTES)
    c3 = wl.REDUCE_CONFIGS["c3_reduce4_64MiB_compress"]
    entries = [(name, lambda n=name: reduce_line(wl.REDUCE_CONFIGS[n]))
               for name in ("c1_copy_4MiB_rot", "c1_copy_4MiB_norot", "c2_reduce2_256MiB_rot",
                            "c2_reduce2_256MiB_norot", "c3_reduce4_64MiB_compress")]
    entries += [
        (c2cold.name, lambda: reduce_line(c2cold)),
        (c2cold.name + "_dstrot", lambda: reduce_line(c2cold, rotate_dst=True)),
        (c3.name + "_dstrot", lambda: reduce_line(c3, rotate_dst=True)),
        ("c4_scatter_47520_rotated", lambda: batch_line(wl.batch_c4(), wl.DEFAULT_ROTATE_BYTES, "rotated")),
        ("c4_scatter_47520_control", lambda: batch_line(wl.batch_c4(), 0, "control")),
        ("c5_mixed_kv_11044_rotated", lambda: batch_line(wl.batch_c5(), wl.DEFAULT_ROTATE_BYTES, "rotated")),
        ("c4_scatter_47520_rotated_dstrot", lambda: batch_line(wl.batch_c4(), wl.DEFAULT_ROTATE_BYTES,
                                                               "rotated_dstrot", BATCH_DST_ROTATE_BYTES)),
        ("c5_mixed_kv_11044_rotated_dstrot", lambda: batch_line(wl.batch_c5(), wl.DEFAULT_ROTATE_BYTES,
                                                                "rotated_dstrot", BATCH_DST_ROTATE_BYTES)),
    ]
    for nbytes in wl.SWEEP_BYTES:
        for rot in (True, False):
            sw = wl.sweep_workload(nbytes, rot)
            entries.append((sw.name, lambda sw=sw: reduce_line(sw, reps=3)))
    # how the reduce-copy scales with the number of sources (64 MiB each, R = 256 MiB)
    for nsrc in (1, 2, 3, 4, 6, 8, 12, 16):
        nw = wl.ReduceWorkload(f"nsweep_N{nsrc}_64MiB", nsrc, 16 << 20, wl.DEFAULT_ROTATE_BYTES)
        entries.append((nw.name, lambda nw=nw: reduce_line(nw)))
    names = [n for n, _ in entries]
    only = [n for n in (args.only or "").split(",") if n]
    unknown = [n for n in only if n not in names]
    if unknown:
        raise SystemExit(f"--only: unknown configuration(s) {unknown}; known: {names}")
    print(json.dumps({"suite_device": device_record(torch, tb)}), flush=True)
    for name, fn in entries:
        if not only or name in only:
            print(json.dumps({"suite": fn()}), flush=True)


# ---------------------------------------------------------------------------
# --baselines: the HIP runtime's own copies on the same inputs
# ---------------------------------------------------------------------------

HIP_MEMCPY_D2D = 3          # hipMemcpyDeviceToDevice: the runtime copies with a kernel
HIP_MEMCPY_D2D_NOCU = 1024  # hipMemcpyDeviceToDeviceNoCU: a copy engine (SDMA), no compute units


def hip_memcpy_fn():
    """hipMemcpyAsync of the HIP runtime torch loaded (the one libtb binds to)."""
    import ctypes
    import re
    with open("/proc/self/maps") as f:
        paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", f.read())))
    if not paths:
        raise RuntimeError("the HIP runtime is not loaded")
    paths.sort(key=lambda q: "torch" not in q)
    fn = ctypes.CDLL(paths[0]).hipMemcpyAsync
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    return fn


def percopy_submit(memcpy, srcs, dsts, sizes, kind, stream_handle):
    """One hipMemcpyAsync per descriptor; returns (seconds spent submitting, OR of the return codes)."""
    rc = 0
    t0 = time.perf_counter()
    for a, d, n in zip(srcs, dsts, sizes):
        rc |= memcpy(d, a, n, kind, stream_handle)
    return time.perf_counter() - t0, rc


def baselines(args, torch, tb, wl):
    """The runtime's device-to-device copy (kernel, and copy engine) on the N = 1
    configurations, and one hipMemcpyAsync per descriptor for the batched ones:
    the per-call path a batched kernel replaces (Mooncake RFC #5041, Motivation)."""
    import numpy as np

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    timer = Timed(torch, tb, stream)
    memcpy = hip_memcpy_fn()
    kinds = ((HIP_MEMCPY_D2D, "hipMemcpyAsync D2D (runtime copy kernel)"),
             (HIP_MEMCPY_D2D_NOCU, "hipMemcpyAsync D2D NoCU (copy engine)"))
    print(json.dumps({"baseline_device": device_record(torch, tb)}), flush=True)

    def copy_line(w, kind, label, reps):
        rs, dst = setup_reduce(torch, w)
        nbytes = w.nfloats * 4
        dp = int(dst.data_ptr())

        def one(i):
            (p,) = rs.pointers(i)
            if memcpy(dp, p, nbytes, kind, sh) != 0:
                raise RuntimeError(f"hipMemcpyAsync failed ({label})")
        means = []
        for rep in range(reps):
            for i in range(-args.warmup, 0):
                one(i)
            ms, _, _ = timer.run([lambda i=i: one(i) for i in range(args.steps)])
            means.append((statistics.mean(ms), min(ms), max(ms)))
        med = sorted(means)[len(means) // 2]
        ok = oracle_reduce_ok([dst], w)
        gbps = w.algorithmic_bytes / (med[0] * 1e-3) / 1e9
        out = {"config": w.name, "method": label, "k": rs.k, "reps": reps, "ms_mean": round(med[0], 5),
               "ms_min": round(med[1], 5), "ms_max": round(med[2], 5), "gbps": round(gbps, 1),
               "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "validated": ok}
        del rs, dst
        torch.cuda.empty_cache()
        return out

    def percopy_line(batch, kind, label, runs=3):
        b = setup_batch(torch, tb, batch, wl.DEFAULT_ROTATE_BYTES)
        pool_base = int(b["pool"].data_ptr())
        dsts = (batch.desc[:, 1].astype(np.int64) + pool_base).tolist()
        sizes = batch.desc[:, 2].astype(np.int64).tolist()
        srcs_per = [(batch.desc[:, 0].astype(np.int64) + b["base"] + r * b["stride"]).tolist() for r in range(b["kb"])]
        walls, submits = [], []
        for i in range(-1, runs):
            r = replica_of(tb, b, i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            sub, rc = percopy_submit(memcpy, srcs_per[r], dsts, sizes, kind, sh)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            if rc != 0:
                raise RuntimeError(f"hipMemcpyAsync failed ({label})")
            if i >= 0:
                walls.append(wall)
                submits.append(sub)
        wall, sub = statistics.median(walls), statistics.median(submits)
        gbps = batch.algorithmic_bytes / wall / 1e9
        out = {"config": batch.name, "method": label, "calls": batch.ncopies, "replicas": b["kb"], "runs": runs,
               "wall_ms": round(wall * 1e3, 3), "host_submit_us_per_call": round(sub / batch.ncopies * 1e6, 3),
               "gbps": round(gbps, 2), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 5),
               "copies_per_s": round(batch.ncopies / wall, 1),
               "validated": oracle_pool_ok([b["pool"]], batch)}
        del b
        torch.cuda.empty_cache()
        return out

    for name in ("c1_copy_4MiB_rot", "c1_copy_4MiB_norot"):
        for kind, label in kinds:
            print(json.dumps({"baseline": copy_line(wl.REDUCE_CONFIGS[name], kind, label, 1)}), flush=True)
    for nbytes in wl.SWEEP_BYTES:
        for rot in (True, False):
            for kind, label in kinds:
                print(json.dumps({"baseline": copy_line(wl.sweep_workload(nbytes, rot), kind, label, 3)}), flush=True)
    for make in (wl.batch_c4, wl.batch_c5):
        batch = make()
        for kind, label in kinds:
            print(json.dumps({"baseline": percopy_line(batch, kind, "one " + label + " per descriptor")}), flush=True)
        del batch


# ---------------------------------------------------------------------------
# --cache-study: what rotation defeats, and what it does not
# ---------------------------------------------------------------------------

def cache_study(args, torch, tb, wl):
    """Per size and SRC_ROTATE_BYTES in {0, 256 MiB, 512 MiB, 1 GiB}: the first
    launch after preparation (cold), the warm mean, and the warm mean with an
    untimed 1 GiB streaming copy before every launch (memory-side cache flushed;
    a labelled variant, not the pages' method).  TransferBench PR #365, Test
    Result and Technical Details."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    timer = Timed(torch, tb, stream)
    MiB = 1 << 20
    fa = torch.empty(128 * MiB, dtype=torch.float32, device="cuda")   # 512 MiB each: a 1 GiB flush copy
    fb = torch.empty_like(fa)
    fa_p, fb_p = int(fa.data_ptr()), int(fb.data_ptr())

    def flush():
        tb.tb_reduce_copy(fb_p, [fa_p], fa.numel(), sh)

    print(json.dumps({"cache_study_device": device_record(torch, tb)}), flush=True)
    shapes = [("copy", 1, 4 * MiB), ("copy", 1, 16 * MiB), ("copy", 1, 64 * MiB), ("reduce2", 2, 256 * MiB),
              ("copy", 1, 512 * MiB)]
    for kind, nsrc, nbytes in shapes:
        for r_mib in (0, 256, 512, 1024):
            w = wl.ReduceWorkload(f"{kind}_{nbytes // MiB}MiB_R{r_mib}MiB", nsrc, nbytes // 4, r_mib * MiB)
            rs, dst = setup_reduce(torch, w)
            dp = int(dst.data_ptr())
            i0 = -args.warmup if args.warmup else 0
            cold, _, _ = timer.run([lambda p=rs.pointers(i0): tb.tb_reduce_copy(dp, p, w.nfloats, sh)])
            for i in range(i0 + 1, 0):
                tb.tb_reduce_copy(dp, rs.pointers(i), w.nfloats, sh)
            warm, _, _ = timer.run([lambda p=rs.pointers(i): tb.tb_reduce_copy(dp, p, w.nfloats, sh)
                                    for i in range(args.steps)])
            # flushed: events bracket only the measured launch
            flushed = []
            for i in range(args.steps):
                flush()
                ms, _, _ = timer.run([lambda p=rs.pointers(i): tb.tb_reduce_copy(dp, p, w.nfloats, sh)])
                flushed.append(ms[0])
            ok = oracle_reduce_ok([dst], w)
            wm, fm = statistics.mean(warm), statistics.mean(flushed)
            gb = w.algorithmic_bytes / 1e9
            print(json.dumps({"cache_study": {
                "config": w.name, "nsrc": nsrc, "bytes_per_buffer": nbytes, "rotate_bytes": r_mib * MiB, "k": rs.k,
                "cold_us": round(cold[0] * 1e3, 2), "warm_us": round(wm * 1e3, 2), "flushed_us": round(fm * 1e3, 2),
                "cold_frac": round(gb / (cold[0] * 1e-3) / HBM_PEAK_GBPS, 4),
                "warm_frac": round(gb / (wm * 1e-3) / HBM_PEAK_GBPS, 4),
                "flushed_frac": round(gb / (fm * 1e-3) / HBM_PEAK_GBPS, 4),
                "warm_over_cold": round(cold[0] / wm, 3), "validated": ok}}), flush=True)
            del rs, dst
            torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# --interference: the batched copy beside a memory-bound neighbour
# ---------------------------------------------------------------------------

def interference(args, torch, tb, wl):
    """The batched copy beside a memory-bound neighbour on a second stream
    (default priority): torch's own copy of 512 MiB (1 GiB of HBM traffic per
    kernel).  C4's batched launches run back to back for as long as 10
    neighbour copies run, uncapped and with the grid capped at 512 and 32
    workgroups (tb_batched_set_max_workgroups); the slowdown of each side.
    Mooncake RFC #5041, Design of #5040: interference with other work, and its
    open question on CU budgets."""
    s_copy = torch.cuda.current_stream()
    s_other = torch.cuda.Stream()
    sh = s_copy.cuda_stream
    timer = Timed(torch, tb, s_copy)
    X = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    Y = torch.empty_like(X)

    def neighbours(n):
        """n neighbour copies on the second stream between two events."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s_other):
            e0.record(s_other)
            for _ in range(n):
                Y.copy_(X)
            e1.record(s_other)
        return e0, e1

    batch = wl.batch_c4()
    b = setup_batch(torch, tb, batch, wl.DEFAULT_ROTATE_BYTES, BATCH_DST_ROTATE_BYTES)

    def copies():
        for i in range(-args.warmup, 0):
            tb.tb_batched_copy(int(batch_desc_for(tb, b, i).data_ptr()), batch.ncopies, sh)
        ds = [batch_desc_for(tb, b, i) for i in range(args.steps)]
        ms, _, _ = timer.run([lambda d=d: tb.tb_batched_copy(int(d.data_ptr()), batch.ncopies, sh) for d in ds])
        return statistics.mean(ms)

    def overlap(cap):
        tb.tb_batched_set_max_workgroups(cap)
        a_ms = copies()
        neighbours(3)
        e0, e1 = neighbours(10)
        torch.cuda.synchronize()
        n_alone = e0.elapsed_time(e1) / 10
        m = int(1.2 * 10 * n_alone / a_ms) + 2
        ds = [batch_desc_for(tb, b, i) for i in range(m)]
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0, h1 = neighbours(10)
        c0.record(s_copy)
        for d in ds:
            tb.tb_batched_copy(int(d.data_ptr()), batch.ncopies, sh)
        c1.record(s_copy)
        torch.cuda.synchronize()
        n_under = h0.elapsed_time(h1) / 10
        c_window = c0.elapsed_time(c1)
        c_under = c_window / m
        e0, e1 = neighbours(10)          # alone again after: the baseline is the faster of the two
        torch.cuda.synchronize()
        n_alone = min(n_alone, e0.elapsed_time(e1) / 10)
        return {"max_workgroups": cap or "none", "copies": m,
                "us_alone": round(a_ms * 1e3, 2), "us_beside_neighbour": round(c_under * 1e3, 2),
                "copy_slowdown": round(c_under / a_ms, 3),
                "gbps_alone": round(batch.algorithmic_bytes / (a_ms * 1e-3) / 1e9, 1),
                "gbps_beside_neighbour": round(batch.algorithmic_bytes / (c_under * 1e-3) / 1e9, 1),
                "neighbour_ms_alone": round(n_alone, 4), "neighbour_ms_beside_copies": round(n_under, 4),
                "neighbour_slowdown": round(n_under / n_alone, 3),
                "copy_window_over_neighbour_window": round(c_window / (n_under * 10), 2)}

    runs = []
    try:
        for cap in (0, 512, 32):
            runs.append(overlap(cap))
    finally:
        tb.tb_batched_set_max_workgroups(0)
    rec = {"neighbour": "torch copy_ of 512 MiB (1 GiB of HBM traffic per kernel) on a second stream",
           "batched_copy": "C4, 47,520 copies", "runs": runs,
           "validated": oracle_pool_ok(pools_written(b, -args.warmup, args.steps), batch)}
    print(json.dumps({"interference": rec}), flush=True)


# ---------------------------------------------------------------------------
# --ring: the descriptor-slot ring's host cost and end-to-end rate
# ---------------------------------------------------------------------------

def ring_study(args, torch, tb, wl):
    """The descriptor-slot ring (Mooncake RFC #5041, Design of #5040,
    "Descriptor slots" and "Host trims"): host nanoseconds per request and per
    copy for submit and poll, and the end-to-end rate of the 47,520-copy and the
    mixed KV batches cut into requests, through staged and direct rings of 32
    slots x 8,192 descriptors; beside them, one tb_batched_copy of the whole
    batch from device memory.  The C calls are made through ctypes directly;
    the ctypes floor (a trivial library call) is reported with them."""
    import ctypes
    import numpy as np

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    lib = tb.lib
    ns = time.perf_counter_ns
    print(json.dumps({"ring_device": device_record(torch, tb)}), flush=True)

    def floor_ns(reps=20000):
        t0 = ns()
        for _ in range(reps):
            lib.tb_batched_set_mode(0)
        return (ns() - t0) / reps

    def one_pass(ring, host, cuts):
        """Submit every request of one batch, then poll the last ticket until
        done.  Returns host ns of the submits made while every slot was free,
        of all submits, per pending poll, the number of polls, and the wall ns."""
        t = ctypes.c_uint64()
        done = ctypes.c_int32()
        base = host.ctypes.data
        free_ns = all_ns = 0
        t0 = ns()
        for j, (a, m) in enumerate(cuts):
            s0 = ns()
            rc = lib.tb_ring_submit(ring, base + 24 * a, m, ctypes.byref(t))
            dt = ns() - s0
            if rc != 0:
                raise tb.TBError("tb_ring_submit", rc)
            all_ns += dt
            if j < 32:
                free_ns += dt
        polls, p_ns = 0, 0
        while True:
            s0 = ns()
            rc = lib.tb_ring_poll(ring, t.value, ctypes.byref(done))
            p_ns += ns() - s0
            polls += 1
            if rc != 0:
                raise tb.TBError("tb_ring_poll", rc)
            if done.value:
                break
        return free_ns, all_ns, p_ns / polls, polls, ns() - t0

    floor = floor_ns()
    for batch in (wl.batch_c4(), wl.batch_c5()):
        b = setup_batch(torch, tb, batch, wl.DEFAULT_ROTATE_BYTES)
        pool_base = int(b["pool"].data_ptr())
        hosts = []
        for r in range(b["kb"]):
            d = batch.desc.astype(np.uint64).copy()
            d[:, 0] += np.uint64(b["base"] + r * b["stride"])
            d[:, 1] += np.uint64(pool_base)
            hosts.append(np.ascontiguousarray(d))
        n = batch.ncopies
        # one launch of the whole batch from device memory, host wall clock to the end
        walls = []
        for i in range(-args.warmup, args.steps):
            torch.cuda.synchronize()
            t0 = ns()
            tb.tb_batched_copy(int(batch_desc_for(tb, b, i).data_ptr()), n, sh)
            stream.synchronize()
            if i >= 0:
                walls.append(ns() - t0)
        ref_us = statistics.median(walls) / 1e3
        print(json.dumps({"ring": {"batch": batch.name, "ncopies": n, "path": "tb_batched_copy, device descriptors",
                                   "wall_us": round(ref_us, 2),
                                   "gbps": round(batch.algorithmic_bytes / (ref_us * 1e-6) / 1e9, 1)}}), flush=True)
        for kind in (tb.TB_RING_STAGED, tb.TB_RING_DIRECT):
            ring = tb.tb_ring_create(32, 8192, kind, sh)
            try:
                for req in (16, 256, 4096, 8192):
                    cuts = [(a, min(req, n - a)) for a in range(0, n, req)]
                    rows = []
                    for i in range(-args.warmup, args.steps):
                        r = one_pass(ring, hosts[replica_of(tb, b, i)], cuts)
                        if i >= 0:
                            rows.append(r)
                    free_n = min(32, len(cuts))
                    free_copies = sum(m for _, m in cuts[:free_n])
                    wall_us = statistics.median([r[4] for r in rows]) / 1e3
                    sub_free = statistics.median([r[0] for r in rows])
                    rec = {"batch": batch.name, "ncopies": n,
                           "path": "ring " + ("direct" if kind == tb.TB_RING_DIRECT else "staged"),
                           "slots": "32 x 8192", "copies_per_request": req, "requests": len(cuts),
                           "submit_ns_per_request_slots_free": round(sub_free / free_n),
                           "submit_ns_per_copy_slots_free": round(sub_free / free_copies, 1),
                           "submit_ns_per_request_all": round(statistics.median([r[1] for r in rows]) / len(cuts)),
                           "poll_ns_pending": round(statistics.median([r[2] for r in rows])),
                           "polls_per_pass": int(statistics.median([r[3] for r in rows])),
                           "ctypes_floor_ns": round(floor),
                           "wall_us": round(wall_us, 2),
                           "gbps": round(batch.algorithmic_bytes / (wall_us * 1e-6) / 1e9, 1),
                           "copies_per_s": round(n / (wall_us * 1e-6), 0)}
                    print(json.dumps({"ring": rec}), flush=True)
                # a poll answered from the ring's record of finished tickets
                t = ctypes.c_uint64()
                done = ctypes.c_int32()
                lib.tb_ring_submit(ring, None, 0, ctypes.byref(t))
                t0 = ns()
                for _ in range(20000):
                    lib.tb_ring_poll(ring, t.value, ctypes.byref(done))
                cached = (ns() - t0) / 20000
            finally:
                tb.tb_ring_destroy(ring)
            print(json.dumps({"ring_poll_cached": {"path": "ring " + ("direct" if kind == tb.TB_RING_DIRECT
                                                                       else "staged"),
                                                   "poll_ns": round(cached), "ctypes_floor_ns": round(floor)}}),
                  flush=True)
        ok = oracle_pool_ok([b["pool"]], batch)
        print(json.dumps({"ring_validated": {"batch": batch.name, "ok": ok}}), flush=True)
        if not ok:
            raise RuntimeError(f"ring copies of {batch.name} differ from the oracle's")
        del b
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# --roofs: what this chip's HBM sustains for reads, writes and their mix
# ---------------------------------------------------------------------------

def roofs(args, torch, tb, wl):
    """What the access patterns allow, from instruments that share no code with
    the library's kernels (libtb_roofs, include/tb_roofs.h; torch's own kernels
    as an outside reference), each beside the library kernel that runs the same
    pattern.  Every rate is the loop rate: the launches queued back to back
    behind the spin gate, one event at each end, divided by the launch count.
      1. streams larger than the 256 MB memory-side cache: read-only (the
         instrument, and torch's sum), write-only (both store policies, the
         library's memset, torch's fill) and a 512 MiB copy;
      2. N + 1 streams of 64 MiB rotated over 4 slices read at once, and N
         streams read with their XOR written to one more (the reduce-copy's
         own pattern with integer work only), against the reduce-copy with N
         sources (N reads, one write, destination rotated the same way);
      3. C4's 47,520 copies cut into <= 4 KiB tiles on the host (the same
         bytes, source replicas and destination pools as the bench step): tile
         copy, destinations written only, sources read only, against the
         batched copy; the same for the copies packed side by side, and for
         C5a's mixed batch.
    Then the launch floor and the host's cost of one call."""
    import numpy as np

    import copy_reduce_amd.roofs as rf
    import oracle
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    MiB = 1 << 20
    print(json.dumps({"roof_device": device_record(torch, tb)}), flush=True)

    def loop_us(fns):
        """Per-launch microseconds of fns (one per iteration, i = 0 .. steps-1)
        run back to back after warmup launches of the same sequence."""
        for fn in fns[:args.warmup]:
            fn()
        ms, _ = run_whole(torch, tb, stream, fns)
        return ms * 1e3 / len(fns)

    def line(kind, label, us, nbytes, **extra):
        gbps = nbytes / (us * 1e-6) / 1e9
        rec = {"kind": kind, "stream": label, "bytes_per_launch": nbytes, "us_per_launch": round(us, 2),
               "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        rec.update(extra)
        print(json.dumps({"roof": rec}), flush=True)

    # ---- 1. single streams above the memory-side cache's size ----
    big = torch.empty(256 * MiB, dtype=torch.float32, device="cuda")           # 1 GiB
    big2 = torch.empty_like(big)
    bp, bp2 = int(big.data_ptr()), int(big2.data_ptr())
    n = args.steps
    line("instrument", "read-only, 1 GiB", loop_us([lambda: rf.tbr_read([bp], 1 << 30, sh)] * n), 1 << 30)
    line("torch", "read-only: torch.sum over 1 GiB (its own reduction kernel)",
         loop_us([lambda: big.sum()] * n), 1 << 30)
    for pol, name in ((rf.TBR_STORE_STREAMING, "nt sc0 sc1"), (rf.TBR_STORE_DEVICE, "sc1")):
        line("instrument", f"write-only, 1 GiB, {name} stores",
             loop_us([lambda pol=pol: rf.tbr_write([bp], 1 << 30, 0x3F800000, pol, sh)] * n), 1 << 30)
    line("library", "write-only: tb_reduce_copy nsrc=0, 1 GiB",
         loop_us([lambda: tb.tb_reduce_copy(bp, [], big.numel(), sh, 0x5A)] * n), 1 << 30)
    line("torch", "write-only: torch fill_ over 1 GiB (its own kernel)",
         loop_us([lambda: big.view(torch.uint8).fill_(0x5A)] * n), 1 << 30)
    half = 512 * MiB
    for pol, name in ((rf.TBR_STORE_STREAMING, "nt sc0 sc1"), (rf.TBR_STORE_DEVICE, "sc1")):
        line("instrument", f"copy 512 MiB, {name} stores, destination alternating between two buffers",
             loop_us([lambda i=i, pol=pol: rf.tbr_copy(bp2 + (i % 2) * half, bp, half, pol, sh)
                      for i in range(n)]), 2 * half)
    line("library", "copy 512 MiB: tb_reduce_copy nsrc=1, destination alternating between two buffers",
         loop_us([lambda i=i: tb.tb_reduce_copy(bp2 + (i % 2) * half, [bp], half // 4, sh) for i in range(n)]),
         2 * half)
    del big, big2
    torch.cuda.empty_cache()

    # ---- 2. N + 1 read streams against the N-source reduce-copy ----
    nb, kslices = 64 * MiB, 4
    bufs = [torch.empty(kslices * nb, dtype=torch.uint8, device="cuda") for _ in range(17)]
    for t in bufs:
        t.fill_(0x3C)
    dsts = torch.empty(kslices * nb, dtype=torch.uint8, device="cuda")
    base = [int(t.data_ptr()) for t in bufs]
    dbase = int(dsts.data_ptr())
    for nsrc in (1, 2, 4, 8, 16):
        k = nsrc + 1
        line("instrument", f"read-only, {k} streams of 64 MiB rotated over 4 slices",
             loop_us([lambda i=i, k=k: rf.tbr_read([b + (i % kslices) * nb for b in base[:k]], nb, sh)
                      for i in range(n)]), k * nb, streams=k)
        # the reduce-copy's own pattern: nsrc streams read, one written (their
        # XOR), with the library's store policy for that source count
        pol, pname = ((rf.TBR_STORE_STREAMING, "nt sc0 sc1") if nsrc <= 2 else (rf.TBR_STORE_NT, "nt"))
        line("instrument", f"{nsrc} streams read, their XOR written to one more ({pname} stores), 64 MiB each, "
             "rotated over 4 slices",
             loop_us([lambda i=i, nsrc=nsrc, pol=pol: rf.tbr_combine([b + (i % kslices) * nb for b in base[:nsrc]],
                                                                    dbase + (i % kslices) * nb, nb, pol, sh)
                      for i in range(n)]), (nsrc + 1) * nb, streams=nsrc + 1, nsrc=nsrc)
        line("library", f"tb_reduce_copy nsrc={nsrc}, 64 MiB per buffer, sources and destination rotated over 4 "
             "slices", loop_us([lambda i=i, nsrc=nsrc: tb.tb_reduce_copy(
                 dbase + (i % kslices) * nb, [b + (i % kslices) * nb for b in base[:nsrc]], nb // 4, sh)
                 for i in range(n)]), (nsrc + 1) * nb, nsrc=nsrc)
    del bufs, dsts
    torch.cuda.empty_cache()

    # ---- 3. C4's pattern: the same bytes as host-cut tiles against the batched copy ----
    for placement, label, batch in (("random_slots", "C4 random_slots", wl.batch_c4_placed("random_slots")),
                                    ("packed", "C4 packed", wl.batch_c4_placed("packed")),
                                    ("c5a", "C5a", wl.batch_c5())):
        b = setup_batch(torch, tb, batch, wl.DEFAULT_ROTATE_BYTES, BATCH_DST_ROTATE_BYTES)
        tiles = {}
        for (sbase, pbase) in b["descs"]:
            t = rf.cut_tiles(batch.desc, sbase, pbase)
            tiles[(sbase, pbase)] = torch.from_numpy(t.view(np.int64)).cuda()
        ntiles = next(iter(tiles.values())).shape[0]

        def tiles_for(i):
            (src,) = tb.tb_rotate_sources([b["base"]], b["stride"], b["kb"], i)
            (pool,) = tb.tb_rotate_sources([b["pbase"]], b["pstride"], b["kp"], i)
            return int(tiles[(src, pool)].data_ptr())
        payload = batch.algorithmic_bytes
        extra = {"placement": placement, "copies": batch.ncopies, "tiles": ntiles, "replicas": b["kb"],
                 "pools": b["kp"]}
        line("library", f"{label}: tb_batched_copy",
             loop_us([lambda d=batch_desc_for(tb, b, i): tb.tb_batched_copy(int(d.data_ptr()), batch.ncopies, sh)
                      for i in range(n)]), payload, **extra)
        for pol, name in ((rf.TBR_STORE_STREAMING, "nt sc0 sc1"), (rf.TBR_STORE_DEVICE, "sc1")):
            line("instrument", f"{label}: tile copy, {name} stores",
                 loop_us([lambda i=i, pol=pol: rf.tbr_tiles_copy(tiles_for(i), ntiles, pol, sh)
                          for i in range(n)]), payload, **extra)
        line("instrument", f"{label}: destinations written only, nt sc0 sc1 stores",
             loop_us([lambda i=i: rf.tbr_tiles_write(tiles_for(i), ntiles, 0xA5A5A5A5, rf.TBR_STORE_STREAMING, sh)
                      for i in range(n)]), payload // 2, **extra)
        line("instrument", f"{label}: sources read only",
             loop_us([lambda i=i: rf.tbr_tiles_read(tiles_for(i), ntiles, sh) for i in range(n)]),
             payload // 2, **extra)
        # the tile copy writes the batch's bytes: check one pool against the oracle
        b["pool_views"][0].fill_(wl.POOL_FILL)
        rf.tbr_tiles_copy(tiles_for(0), ntiles, rf.TBR_STORE_STREAMING, sh)
        torch.cuda.synchronize()
        exp = np.full(batch.pool_bytes, wl.POOL_FILL, dtype=np.uint8)
        oracle.ref_batch(exp, batch.payload, batch.desc)
        ok = oracle.first_mismatch(b["pool_views"][0].cpu().numpy(), exp) == -1
        print(json.dumps({"roof_check": {"placement": placement, "tile_copy_equals_oracle": ok}}), flush=True)
        if not ok:
            raise RuntimeError(f"the tile copy of {label} differs from the oracle")
        del b, tiles, exp
        torch.cuda.empty_cache()

    # Launch floor: a copy of 64 floats (one workgroup, next to no work) and
    # C1's 4 MiB copy, 20 launches back to back (one event at each end) and by
    # each launch's own start and stop events.
    n1 = 1 << 20
    floor_buf = torch.empty(9 * n1, dtype=torch.float32, device="cuda")      # 8 sources of 4 MiB + dst
    ap = int(floor_buf.data_ptr())
    bp2 = ap + 8 * 4 * n1
    for label, nf in (("copy of 256 B (one workgroup)", 64), ("copy of 4 MiB (C1 size)", n1)):
        fns = [lambda j=j, nf=nf: tb.tb_reduce_copy(bp2, [ap + (j % 8) * 4 * n1], nf, sh) for j in range(20)]
        for fn in fns[:args.warmup]:
            fn()
        loop_ms, _ = run_whole(torch, tb, stream, fns)
        ev_ms, _ = run_launch_events(torch, tb, stream, fns)
        print(json.dumps({"launch_floor": {"launch": label, "launches": len(fns),
                                           "us_per_launch_back_to_back": round(loop_ms * 1e3 / len(fns), 2),
                                           "us_by_own_launch_events": round(statistics.mean(ev_ms) * 1e3, 2)}}),
              flush=True)

    # Host cost of one call: 200 tb_reduce_copy calls of 64 floats enqueued
    # while the spin gate holds the stream (so no call waits for the GPU),
    # timed on the host through this binding (median of 3 rounds).
    for nsrc in (1, 2, 4, 8, 16):
        ptrs = [ap + 4096 * k for k in range(nsrc)]
        per_call = []
        for _ in range(3):
            torch.cuda.synchronize()
            tb.tb_spin_gate_arm(GATE_TIMEOUT_MS, sh)
            t0 = time.perf_counter()
            for _ in range(200):
                tb.tb_reduce_copy(bp2, ptrs, 64, sh)
            t1 = time.perf_counter()
            tb.tb_spin_gate_release()
            torch.cuda.synchronize()
            if tb.tb_spin_gate_status() != tb.TB_OK:
                raise RuntimeError("spin gate timed out: the calls were not gated")
            per_call.append((t1 - t0) / 200)
        print(json.dumps({"host_enqueue": {"call": f"tb_reduce_copy nsrc={nsrc}, 64 floats", "calls": 200,
                                           "us_per_call": round(statistics.median(per_call) * 1e6, 2)}}), flush=True)


def scatter_study(args, torch, tb, wl):
    """What C4's destination pattern costs: the same 47,520 copies (sizes,
    source stream, one launch each) under five destination placements, from
    C4's random 16 KiB slots to destinations packed like the sources.  Per
    placement: the kernel's duration by its own launch events and the
    back-to-back rate, over K_b rotated source replicas."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    print(json.dumps({"scatter_device": device_record(torch, tb)}), flush=True)
    for placement in wl.C4_PLACEMENTS:
        batch = wl.batch_c4_placed(placement)
        b = setup_batch(torch, tb, batch, wl.DEFAULT_ROTATE_BYTES)

        def bc(i):
            d = batch_desc_for(tb, b, i)
            return lambda: tb.tb_batched_copy(int(d.data_ptr()), batch.ncopies, sh)
        for i in range(-args.warmup, 0):
            bc(i)()
        fns = [bc(i) for i in range(args.steps)]
        loops, kernels = [], []
        for _ in range(3):
            loop_ms, _ = run_whole(torch, tb, stream, fns)
            ev_ms, _ = run_launch_events(torch, tb, stream, fns)
            loops.append(loop_ms / len(fns))
            kernels.append(statistics.mean(ev_ms))
        km, lm = statistics.median(kernels), statistics.median(loops)
        nbytes = batch.algorithmic_bytes
        print(json.dumps({"scatter": {
            "placement": placement, "copies": batch.ncopies, "payload_bytes": batch.total_bytes, "kb": b["kb"],
            "pool_span_bytes": int((batch.desc[:, 1] + batch.desc[:, 2]).max()),
            "kernel_us": round(km * 1e3, 2), "kernel_frac_of_peak": round(nbytes / (km * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "loop_us_per_launch": round(lm * 1e3, 2),
            "loop_frac_of_peak": round(nbytes / (lm * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "validated": oracle_pool_ok([b["pool"]], batch)}}), flush=True)
        del b
        torch.cuda.empty_cache()


def misaligned_study(args, torch, tb, wl):
    """The reduce-copy when its sources disagree with dst modulo 16 (the
    unaligned path) against aligned sources: 256 MiB per buffer, 1-16
    sources, every source 0, 4 or 8 bytes past a 16-byte boundary while dst
    sits on one.  Then the batched copy over C4's copies with every source
    shifted by 0, 1, 2, 4 or 8 bytes.  Kernel time from the launches' own events, mean of 10 after
    3 warmups; every result is checked against the oracle (every element of dst,
    every byte of the pool)."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    n = 64 << 20
    print(json.dumps({"misaligned_device": device_record(torch, tb)}), flush=True)
    gen = torch.Generator(device="cuda").manual_seed(17)
    for nsrc in (1, 2, 4, 8, 16):
        srcs = [torch.rand(n + 16, device="cuda", generator=gen) for _ in range(nsrc)]
        dst = torch.empty(n + 16, device="cuda")
        dp = int(dst.data_ptr())
        for off_bytes in (0, 4, 8):
            k = off_bytes // 4
            ptrs = [int(x.data_ptr()) + off_bytes for x in srcs]
            fns = [lambda: tb.tb_reduce_copy(dp, ptrs, n, sh)] * args.steps
            for _ in range(args.warmup):
                fns[0]()
            ms, _ = run_launch_events(torch, tb, stream, fns)
            m = statistics.mean(ms)
            ok = oracle_reduce_ok([dst[:n]], srcs=[x[k:k + n] for x in srcs])
            print(json.dumps({"misaligned": {
                "nsrc": nsrc, "bytes_per_buffer": n * 4, "source_offset_bytes": off_bytes,
                "path": "vector" if off_bytes == 0 else "unaligned",
                "kernel_us": round(m * 1e3, 2),
                "frac_of_peak": round((nsrc + 1) * n * 4 / (m * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "validated": ok}}),
                  flush=True)
        del srcs, dst
        torch.cuda.empty_cache()

    # the batched copy: C4's copies with every source shifted by 0-8 bytes
    # (destinations unchanged), so source and destination disagree modulo 16
    import numpy as np
    from copy_reduce_amd.torch_api import make_desc
    batch = wl.batch_c4()
    src = torch.zeros(batch.src_bytes + 4096, dtype=torch.uint8, device="cuda")
    src[:batch.src_bytes] = torch.from_numpy(batch.payload).cuda()
    pool = torch.full((batch.pool_bytes,), wl.POOL_FILL, dtype=torch.uint8, device="cuda")
    for shift in (0, 1, 2, 4, 8):
        d = batch.desc.copy()
        d[:, 0] += np.uint64(shift)
        desc = make_desc(d, int(src.data_ptr()), int(pool.data_ptr()))
        fns = [lambda: tb.tb_batched_copy(int(desc.data_ptr()), batch.ncopies, sh)] * args.steps
        for _ in range(args.warmup):
            fns[0]()
        ms, _ = run_launch_events(torch, tb, stream, fns)
        m = statistics.mean(ms)
        ok = oracle_pool_ok([pool], batch, src_shift=shift)
        print(json.dumps({"misaligned_batch": {
            "copies": batch.ncopies, "source_shift_bytes": shift, "kernel_us": round(m * 1e3, 2),
            "frac_of_peak": round(batch.algorithmic_bytes / (m * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "validated": ok}}), flush=True)


def calibrate_copy(torch, tb):
    """A plain copy of exactly 268,435,456 bytes read and 268,435,456 written per launch."""
    nbytes = 256 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sh = torch.cuda.current_stream().cuda_stream
    for _ in range(10):
        tb.tb_reduce_copy(int(dst.data_ptr()), [int(src.data_ptr())], nbytes // 4, sh)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "tb_reduce_copy nsrc=1", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": 10}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--suite", action="store_true", help="also time every configuration (C1-C5, sweep)")
    ap.add_argument("--baselines", action="store_true",
                    help="only time the HIP runtime's own copies (copy kernel, copy engine, one call per "
                         "descriptor) on the same inputs, then exit")
    ap.add_argument("--interference", action="store_true",
                    help="only time C4's batched copy alone and beside a memory-bound neighbour (torch's 512 MiB "
                         "copy on a second stream), uncapped and with its grid capped, then exit")
    ap.add_argument("--cpu-suite", action="store_true",
                    help="only time the oracle on one host core for every configuration (no GPU), then exit")
    ap.add_argument("--ring", action="store_true",
                    help="only time the descriptor-slot ring (host submit/poll cost, end-to-end rate), then exit")
    ap.add_argument("--roofs", action="store_true",
                    help="only time write-only, read-mostly and copy streams larger than the memory-side cache, then exit")
    ap.add_argument("--cache-study", action="store_true",
                    help="only run the rotation / cold / warm / flushed study over sizes and SRC_ROTATE_BYTES, then exit")
    ap.add_argument("--scatter-study", action="store_true",
                    help="only time C4's copies under five destination placements (random slots to packed), then exit")
    ap.add_argument("--misaligned", action="store_true",
                    help="only time the reduce-copy with sources 0, 4 or 8 bytes off dst's 16-byte alignment "
                         "(1-16 sources of 256 MiB) and C4's batched copies with sources shifted 0-8 bytes, then exit")
    ap.add_argument("--only", default="",
                    help="comma-separated suite configurations to run (implies --suite; the bench line is skipped)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB copy (tb_reduce_copy, one source) 10 times: the known-size "
                         "kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE into HBM bytes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the transfer path measured here runs on one GPU's HBM (sharding across GPUs is designed, not built).",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    if args.cpu_suite:
        import workloads as wl
        cpu_baseline_suite(args, wl)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU: the HIP path has no CPU fallback", file=sys.stderr, flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)
    import copy_reduce_amd as tb
    import workloads as wl

    if args.calibrate_copy:
        calibrate_copy(torch, tb)
        return
    if args.baselines:
        baselines(args, torch, tb, wl)
        return
    if args.cache_study:
        cache_study(args, torch, tb, wl)
        return
    if args.roofs:
        roofs(args, torch, tb, wl)
        return
    if args.interference:
        interference(args, torch, tb, wl)
        return
    if args.ring:
        ring_study(args, torch, tb, wl)
        return
    if args.scatter_study:
        scatter_study(args, torch, tb, wl)
        return
    if args.misaligned:
        misaligned_study(args, torch, tb, wl)
        return
    if args.suite or args.only:
        suite(args, torch, tb, wl)
        torch.cuda.empty_cache()
        if args.only:
            return
    main_line(args, torch, tb, wl)


if __name__ == "__main__":
    main()
