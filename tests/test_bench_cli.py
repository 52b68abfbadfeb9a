"""bench.py's command-line contract on a machine without a GPU: one GPU only,
argument checks, and a loud failure when no GPU is present (there is no CPU
fallback for the measured path)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    if env_extra:
        env.update(env_extra)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_refuses_other_gpu_counts(n):
    r = _run(["--gpus", n])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_refuses_a_distributed_launch():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_rejects_bad_step_counts():
    assert _run(["--steps", "0"]).returncode == 2
    assert _run(["--warmup", "-1"]).returncode == 2


def test_fails_loudly_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run(["--no-cpu-baseline"])
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
    assert '"metric"' not in r.stdout


def _ignored_by_gpu_snapshot(rel):
    """True if a line of .gpurunignore (tar exclude patterns) drops `rel`."""
    import fnmatch
    path = os.path.join(ROOT, ".gpurunignore")
    if not os.path.exists(path):
        return False
    parts = rel.split("/")
    for pat in open(path).read().split():
        if pat.startswith("./"):
            p = pat[2:].rstrip("/")
            if any(fnmatch.fnmatch("/".join(parts[:i + 1]), p) for i in range(len(parts))):
                return True
        elif any(fnmatch.fnmatch(x, pat) for x in parts):
            return True
    return False


def test_counter_summary_travels_with_the_tree():
    """bench.py reads profiles/traffic.json for the roofline's HBM traffic; a GPU
    run sees the tree minus the ignore list, so that file must not be on it.
    While its source hash matches the kernels, both kernels have figures."""
    import importlib.util
    assert not _ignored_by_gpu_snapshot("profiles/traffic.json")
    assert not _ignored_by_gpu_snapshot("copy_reduce_amd/csrc/tb_kernels.hip")
    assert _ignored_by_gpu_snapshot("gpurun_out/x.log")
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    if bench._traffic("reduce_copy") is None:
        pytest.skip("the kernels changed since the counters were taken (traffic is reported as null)")
    assert bench._traffic("batched_copy") > 0
