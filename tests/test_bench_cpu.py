"""bench.py host behaviour that needs no GPU: it measures one GPU only and
refuses a multi-GPU run with a message (no distributed path is timed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "1"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_exits_with_a_message():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2", "RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
