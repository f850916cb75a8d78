"""Parity of the low-latency path (ep_dispatch_ll, ep_combine_ll, called
through the C ABI binding) with the CPU oracle: bit-exact counts, slots,
source tokens, FP8 codes and scales (or BF16 rows); rows no pair takes are
left untouched; combine within 1 bf16 ulp."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from checks import bf16_ulp_diff
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu

SENT_Q = 0x5A          # receive bytes of rows no pair takes
SENT_SC = -7.0
SENT_SRC = -99
NAN_BF16 = 0x7FC0      # expert outputs of rows no pair takes: reading one would show


def say(*a):
    print(*a, flush=True)


def run_ll(w, idx, wt, x, cap, recv_dtype="fp8"):
    cfg = ep.Config.of(w)
    nrows = w.E * cap
    dev = "cuda"
    if recv_dtype == "fp8":
        recv = torch.full((nrows, w.H), SENT_Q, dtype=torch.uint8, device=dev)
        sc = torch.full((nrows, w.H // 128), SENT_SC, dtype=torch.float32, device=dev)
    else:
        recv = torch.full((nrows, w.H), 0x1234, dtype=torch.int16, device=dev).view(torch.bfloat16)
        sc = None
    src = torch.full((nrows,), SENT_SRC, dtype=torch.int32, device=dev)
    r = ep.dispatch_ll(cfg, to_dev(x, torch.bfloat16), to_dev(idx), cap, recv_dtype, recv, sc, recv_src=src)
    # expert outputs: oracle-independent synthetic rows where a pair landed, NaN elsewhere
    torch.cuda.synchronize()
    slot = to_host(r["slot"])
    yrows = W.gen_y(w, nrows=max(1, int((slot >= 0).sum())))
    y = np.full((nrows, w.H), NAN_BF16, np.uint16)
    taken = slot[slot >= 0]
    y[np.sort(taken)] = yrows[: taken.size]
    out = ep.combine_ll(cfg, cap, to_dev(y, torch.bfloat16), r["slot"], to_dev(wt))
    torch.cuda.synchronize()
    res = {k: to_host(v) for k, v in r.items() if v is not None}
    res["out"] = to_host(out)
    res["y"] = y
    return res


def check_ll(w, idx, wt, x, cap, g, recv_dtype="fp8"):
    nrows = w.E * cap
    L = oracle.ll_layout(idx, w.E, cap, src=np.full(nrows, SENT_SRC, np.int32))
    assert np.array_equal(g["count"], L["count"])
    assert np.array_equal(g["slot"], L["slot"])
    assert np.array_equal(g["src"], L["src"])
    if recv_dtype == "fp8":
        q, s = oracle.dispatch_fp8(x, L["slot"], nrows, np.full((nrows, w.H), SENT_Q, np.uint8),
                                   np.full((nrows, w.H // 128), SENT_SC, np.float32))
        assert np.array_equal(g["recv"], q)
        assert np.array_equal(g["scales"].view(np.uint32), s.view(np.uint32))
    else:
        r = oracle.dispatch_bf16(x, L["slot"], nrows, np.full((nrows, w.H), 0x1234, np.uint16))
        assert np.array_equal(g["recv"], r)
    ref = oracle.combine(g["y"], L["slot"], wt)
    d = bf16_ulp_diff(g["out"], ref)
    say("combine_ll: %d of %d differ, max %d ulp; rows taken %d of %d" % (
        (d > 0).sum(), d.size, d.max(), (L["slot"] >= 0).sum(), L["slot"].size))
    assert d.max() <= 1


@pytest.mark.parametrize("name,cap", [("decode", 128), ("decode", 3), ("tiny", 64), ("tiny", 5)])
def test_ll_routed(name, cap):
    w = W.CONFIGS[name]
    say("ll", name, "cap", cap, w)
    lg, x = W.gen_logits(w), W.gen_x(w)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    g = run_ll(w, idx, wt, x, cap)
    check_ll(w, idx, wt, x, cap, g)


def test_ll_bf16():
    w = W.DECODE.replace(H=2048)
    say("ll bf16", w)
    lg, x = W.gen_logits(w), W.gen_x(w)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    g = run_ll(w, idx, wt, x, 16, "bf16")
    check_ll(w, idx, wt, x, 16, g, "bf16")


def test_ll_unrouted_and_repeated():
    w = W.Workload("ll_holes", T=300, H=512, E=24, G=4, TG=4, k=5, R=4, seed=21)
    say("ll holes", w)
    rng = np.random.default_rng(21)
    idx = rng.integers(0, w.E, size=(w.T, w.k)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    idx[rng.random(idx.shape) < 0.03] = w.E + 1
    wt = rng.random((w.T, w.k)).astype(np.float32)
    x = W.gen_x(w)
    for cap in (7, 300):
        g = run_ll(w, idx, wt, x, cap)
        check_ll(w, idx, wt, x, cap, g)


@pytest.mark.parametrize("w,cap", [
    (W.Workload("ll_max", T=1024, H=1024, E=256, G=8, TG=4, k=8, R=32, seed=22), 40),   # T*k = 8192
    (W.Workload("ll_k32", T=256, H=256, E=1024, G=64, TG=8, k=32, R=64, m=4, seed=23), 16),
    (W.Workload("ll_h128", T=77, H=128, E=16, G=4, TG=2, k=4, R=4, seed=24), 9),
    (W.Workload("ll_one", T=1, H=7168, E=256, G=8, TG=4, k=8, R=32, seed=25), 1),
])
def test_ll_edge_shapes(w, cap):
    say("ll edge", w, "cap", cap)
    lg, x = W.gen_logits(w), W.gen_x(w)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    g = run_ll(w, idx, wt, x, cap)
    check_ll(w, idx, wt, x, cap, g)


def test_ll_zero_tokens_writes_counts():
    w = W.DECODE.replace(T=0)
    cfg = ep.Config.of(w)
    cnt = torch.full((w.E,), 5, dtype=torch.int32, device="cuda")
    r = ep.dispatch_ll(cfg, torch.empty((0, w.H), dtype=torch.bfloat16, device="cuda"),
                       torch.empty((0, w.k), dtype=torch.int32, device="cuda"), 4, recv_count=cnt)
    torch.cuda.synchronize()
    assert to_host(r["count"]).tolist() == [0] * w.E


def test_ll_route_on_gpu_end_to_end():
    # the GPU's own routing feeds the low-latency path (decode workload)
    w = W.DECODE
    cfg = ep.Config.of(w)
    lg, x = W.gen_logits(w), W.gen_x(w)
    idx, wt = ep.route(cfg, to_dev(lg))
    g = run_ll(w, to_host(idx), to_host(wt), x, w.T)
    oi, ow = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    assert np.array_equal(to_host(idx), oi)
    check_ll(w, oi, ow, x, w.T, g)
