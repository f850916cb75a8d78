"""bench.py on the CPU: it refuses more than one GPU with a message and a
non-zero status, before touching a GPU, and its rule for the number of
rotating buffer copies keeps every step's inputs out of the caches."""
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


def test_warm_x_is_refused_outside_the_normal_path():
    r = run("--path", "ll", "--warm-x")
    assert r.returncode != 0
    assert "--warm-x" in r.stderr and r.stdout == ""


def test_help_lists_the_paths():
    r = run("--help")
    assert r.returncode == 0
    for word in ("--path", "--config", "--steps", "--warmup", "--gpus"):
        assert word in r.stdout


def test_buffer_copies_keep_every_step_cold():
    # enough copies that >= 512 MB of cache-allocated data (logits, x,
    # scales, index arrays) and >= 2 GiB of traffic lie between two uses of
    # a copy, so no step finds its inputs in the 256 MB Infinity Cache
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    got = {}
    for w in (W.TINY, W.DECODE, W.PREFILL, W.LARGE):
        touched = w.bytes_route() + w.bytes_layout() + w.bytes_dispatch_fp8() + w.bytes_combine()
        cached = bench.cached_bytes(w, w.nrows)
        n = bench.buffer_sets(0, touched, touched, cached)
        got[w.name] = n
        assert 4 <= n <= 256
        if n < 256 and n * touched <= (48 << 30):
            assert (n - 1) * cached >= 512 << 20 and (n - 1) * touched >= 2 << 30
    assert got == {"tiny": 256, "decode": 244, "prefill": 9, "large": 4}
    assert bench.buffer_sets(3, 1, 1, 1) == 3  # --sets N wins
