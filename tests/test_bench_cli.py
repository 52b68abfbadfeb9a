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


def test_counter_summary_matches_the_kernels():
    """bench.py reads profiles/traffic.json for the roofline's HBM traffic and
    reports it only while the file's kernel-source hash matches the kernels;
    while it does, both kernels have figures."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    if bench._traffic("reduce_copy") is None:
        pytest.skip("the kernels changed since the counters were taken (traffic is reported as null)")
    assert bench._traffic("reduce_copy") > 0
    assert bench._traffic("batched_copy") > 0
