"""bench.py's argument handling, on the CPU: the refusals happen before any
device is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_layout_applies_to_the_dense_product_only():
    r = run("--sparse", "--layout", "nt")
    assert r.returncode == 2 and "dense product only" in r.stderr


def test_unknown_layout_is_an_argument_error():
    r = run("--layout", "xy")
    assert r.returncode == 2 and "--layout" in r.stderr
