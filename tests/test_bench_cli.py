"""bench.py's command line without a GPU: a request for more than one GPU is
refused with a message (the layer is built for one GPU), before anything
touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_workload_option():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    assert "--workload" in r.stdout and "--steps" in r.stdout and "--warmup" in r.stdout
