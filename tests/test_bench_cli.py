"""bench.py's command line on the CPU: the measurement is one GPU's share of the ring, so a request
for several GPUs ends at once with a message and exit status 2 (before anything touches a GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_several_gpus_are_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "more than one GPU" in r.stderr
    assert r.stdout == ""


def test_a_distributed_launch_is_refused():
    r = _run(["--steps", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr
