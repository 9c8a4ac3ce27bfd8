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


def test_bench_sharding_matches_the_oracle_layouts():
    """bench.py shards its inputs with its own numpy reshapes; each layout must put token
    oracle.shard_positions(S, P, layout)[i, r] at shard i, row r, or the timed masks would be wrong."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench
    import oracle

    B, H, D = 2, 3, 2
    for S, P in ((48, 4), (64, 8), (24, 2)):
        x = np.arange(B * S * H * D, dtype=np.int64).reshape(B, S, H, D)
        for layout in ("contiguous", "striped", "zigzag"):
            got = bench.shard_np(x, P, layout)
            pos = oracle.shard_positions(S, P, layout)
            want = np.ascontiguousarray(x[:, pos.reshape(-1)].reshape(B, P, S // P, H, D).transpose(1, 0, 2, 3, 4))
            assert got.shape == want.shape
            assert np.array_equal(got, want), (S, P, layout)
