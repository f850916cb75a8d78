"""bench.py's command line on the CPU: it refuses more than one GPU with a
message and a non-zero status, before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_paths():
    r = run("--help")
    assert r.returncode == 0
    for word in ("--path", "--config", "--steps", "--warmup", "--gpus"):
        assert word in r.stdout
