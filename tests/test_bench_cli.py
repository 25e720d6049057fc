"""bench.py's command line on the CPU: runs on more than one GPU, and empty timed
regions, are refused with a message before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2 and "single GPU" in r.stderr and not r.stdout


def test_a_distributed_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _bench(env=env)
    assert r.returncode == 2 and "single GPU" in r.stderr and not r.stdout


def test_empty_timed_region_is_refused():
    r = _bench("--steps", "0")
    assert r.returncode == 2 and "--steps" in r.stderr and not r.stdout
