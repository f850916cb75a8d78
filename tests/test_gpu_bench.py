"""bench.py's step runners in this process, at the small workload: the record
of every path carries the fields its JSON line promises (metric, value,
unit, steps, ms_per_step, config, ...; the normal path also its roofline,
CPU baseline, input provenance and parity record), and the normal path's
own parity check of its buffer set 0 against the oracle passes; the launch
probe runs and reports every probe."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

LINE = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config")


def say(*a):
    print(*a, flush=True)


def args_for(*argv):
    old = sys.argv
    sys.argv = ["bench.py", *argv]
    try:
        return bench.parse()
    finally:
        sys.argv = old


def check_line(rec, steps):
    for key in LINE:
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == steps and rec["data"] == "synthetic"
    assert rec["value"] > 0 and rec["ms_per_step"] > 0


@pytest.mark.parametrize("recv_dtype", ["fp8", "bf16"])
def test_normal_path_record(recv_dtype):
    say("bench normal path, tiny,", recv_dtype)
    a = args_for("--steps", "2", "--warmup", "1", "--sets", "2", "--cpu-seconds", "0.4", "--recv-dtype", recv_dtype)
    rec = bench.run_normal(a, W.TINY)
    check_line(rec, 2)
    for key in ("roofline", "cpu_baseline", "parity", "kernels", "inputs", "graph_step_us"):
        assert key in rec, key
    assert rec["parity"]["verdict"] == "pass", rec["parity"]
    r = rec["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == bench.HBM_PEAK_GBS and r["achieved"] > 0 and 0 < r["frac"]
    c = rec["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["one_thread"]["cores"] == 1
    assert rec["config"]["buffer_sets"] == 2 and rec["config"]["workload"] == "tiny"


def test_normal_path_with_warm_x():
    say("bench normal path, tiny, x shared between the buffer sets")
    a = args_for("--steps", "2", "--warmup", "1", "--sets", "3", "--warm-x", "--no-cpu-baseline")
    rec = bench.run_normal(a, W.TINY)
    check_line(rec, 2)
    assert rec["config"]["x"].startswith("one copy shared")


@pytest.mark.parametrize("recv_dtype", ["fp8", "bf16"])
def test_low_latency_record(recv_dtype):
    say("bench low-latency path, tiny,", recv_dtype)
    a = args_for("--path", "ll", "--steps", "2", "--warmup", "1", "--sets", "2", "--recv-dtype", recv_dtype)
    rec = bench.run_ll(a, W.TINY)
    check_line(rec, 2)
    assert rec["higher_is_better"] is False and rec["unit"].startswith("us")


def test_dedup_record():
    say("bench deduplicated path, tiny")
    rec = bench.run_dedup(args_for("--path", "dedup", "--steps", "2", "--warmup", "1", "--sets", "2"), W.TINY)
    check_line(rec, 2)
    assert 0 < rec["rank_rows_per_token"] <= W.TINY.k


def test_overlap_record():
    say("bench overlap path, tiny")
    a = args_for("--path", "overlap", "--steps", "2", "--warmup", "1", "--sets", "2", "--cus", "32", "--gemm-n", "1024")
    rec = bench.run_overlap(a, W.TINY)
    assert rec["budgets"] and rec["budgets"][0]["comm_cus"] == 32
    assert rec["value"] > 0 and rec["full_gpu"]["dc_us"] > 0


def test_launch_probe_record(capsys):
    # the launch floors and the routing kernel's memory pattern, beside
    # ep_route and ep_route_layout, at the prefill shape
    say("bench launch probe")
    assert bench.launch_probe(args_for("--launch-probe", "--steps", "3")) == 0
    rec = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    names = set(rec["probes"])
    for key in ("empty_256x1024_8KiB", "empty_1024x256", "empty_57344x64", "token_rows_16_per_wg",
                "token_rows_4_per_wg", "ep_route", "ep_route_layout"):
        assert key in names, key
    assert all(v["median_us"] > 0 for v in rec["probes"].values())
