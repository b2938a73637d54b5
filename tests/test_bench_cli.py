"""The benchmark's command-line contract that needs no GPU: more than one
GPU is refused with a message before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    res = _run("--gpus", "2")
    assert res.returncode != 0
    assert "one GPU only" in res.stderr, res.stderr
    assert res.stdout == ""


def test_distributed_launch_is_refused_too():
    env = dict(os.environ, WORLD_SIZE="2")
    res = _run(env=env)
    assert res.returncode != 0 and res.stdout == ""
