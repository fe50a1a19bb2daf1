"""The benchmark's command-line contract, checked on the CPU: one GPU only, no
silent CPU fallback, and the CPU baseline's fields."""

import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU only" in r.stderr
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "WORLD_SIZE 4" in r.stderr


def test_no_gpu_means_no_measurement():
    if torch.cuda.is_available():
        return
    r = _run(["--steps", "1", "--warmup", "0"])
    assert r.returncode == 1 and "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench

    g = torch.Generator().manual_seed(0)
    d = {"x": torch.randn(128, 256, generator=g).to(torch.bfloat16),
         "w": (torch.randn(256, 256, generator=g) * 0.02).to(torch.bfloat16)}
    out = bench.cpu_baseline_dense(d, min_seconds=0.0, max_steps=2)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] == len(os.sched_getaffinity(0))
    assert out["cpu_model"] and out["cpu_model"] != "unknown"
    assert out["sample"].startswith("1 dense step(s)")


def test_rotated_copies_exceed_the_last_level_cache():
    sys.path.insert(0, ROOT)
    import bench

    for nbytes in (4096 * 7168 * 2, 7168 * 7168 * 2, 16384 * 7168 * 2, 7168 * 18432 * 2):
        n = bench._copies(nbytes, 2)
        assert n >= 2 and n * nbytes > bench.LLC_BYTES
