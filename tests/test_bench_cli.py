"""Host-side contract of bench.py: it measures one GPU and refuses more, before
touching a device (the forward pass shards over (batch, head) with no
communication, so a multi-GPU run is one process per GPU, outside the bench)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_world_size_above_one_is_refused():
    r = _run(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr
