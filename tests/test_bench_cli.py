"""The benchmark's command line: one GPU only, refused before anything
touches a device (runs on the CPU)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_a_distributed_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="8")
    r = _bench("--gpus", "1", env=env)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_help_names_the_workload_flag():
    r = _bench("--help")
    assert r.returncode == 0 and "--workload" in r.stdout and "--steps" in r.stdout
