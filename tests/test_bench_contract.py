"""bench.py's command-line contract that needs no GPU: a request for more than
one GPU (by flag or by a distributed launcher's WORLD_SIZE) ends with exit code
2 and a message saying the benchmark runs on one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "4", "--steps", "5", "--warmup", "1"])
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU" in r.stdout


def test_distributed_launch_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU" in r.stdout
