"""The library's calls inside a captured HIP graph (torch.cuda.graph): every
replay gives the eager run's bits, with eager work that overwrites the
outputs between replays.  The calls neither allocate nor clear memory, so
they capture as plain kernel nodes."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import workloads as W
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _capture_and_check(run, outputs, nrep=3):
    run()
    torch.cuda.synchronize()
    ref = [to_host(t).copy() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(nrep):
        for t in outputs:                      # eager work between replays
            t.view(torch.uint8).fill_(0x5A + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs, ref):
            assert np.array_equal(to_host(a), b), "replay %d differs" % rep
    say("graph: %d replays bit-identical to the eager run" % nrep)


def test_normal_step_in_graph():
    w = W.PREFILL.replace(T=1024)
    cfg = ep.Config.of(w)
    lg = to_dev(W.gen_logits(w))
    x = to_dev(W.gen_x(w), torch.bfloat16)
    y = to_dev(W.gen_y(w), torch.bfloat16)
    i32 = dict(dtype=torch.int32, device="cuda")
    idx, wt = torch.empty((w.T, w.k), **i32), torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    lay = dict(cnt=torch.empty(w.E, **i32), ntok_rank=torch.empty(w.R, **i32), off=torch.empty(w.E + 1, **i32),
               slot=torch.empty((w.T, w.k), **i32), recv_token=torch.empty(w.nrows, **i32))
    ws = torch.empty(ep.layout_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    recv = torch.empty((w.nrows, w.H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((w.nrows, w.H // 128), dtype=torch.float32, device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")

    def run():
        ep.route(cfg, lg, idx, wt)
        ep.get_layout(cfg, idx, lay, ws)
        ep.dispatch(cfg, x, lay["slot"], "fp8", recv, sc)
        ep.combine(cfg, y, lay["slot"], wt, out)

    _capture_and_check(run, [idx, wt, *lay.values(), recv, sc, out])


def test_low_latency_and_dedup_steps_in_graph():
    w = W.DECODE
    cfg = ep.Config.of(w)
    cap = w.T
    lg = to_dev(W.gen_logits(w))
    x = to_dev(W.gen_x(w), torch.bfloat16)
    i32 = dict(dtype=torch.int32, device="cuda")
    idx, wt = torch.empty((w.T, w.k), **i32), torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    nr = w.E * cap
    ll = dict(recv=torch.zeros((nr, w.H), dtype=torch.uint8, device="cuda"),
              scales=torch.zeros((nr, w.H // 128), dtype=torch.float32, device="cuda"),
              count=torch.empty(w.E, **i32), src=torch.full((nr,), -1, **i32), slot=torch.empty((w.T, w.k), **i32))
    yll = torch.randn((nr, w.H), device="cuda").to(torch.bfloat16)
    out_ll = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    lay = dict(cnt=torch.empty(w.E, **i32), ntok_rank=torch.empty(w.R, **i32), off=torch.empty(w.E + 1, **i32),
               slot=torch.empty((w.T, w.k), **i32))
    ws = torch.empty(ep.layout_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    rl = dict(rank_count=torch.empty(w.R, **i32), rank_offset=torch.empty(w.R + 1, **i32),
              rank_slot=torch.empty((w.T, w.k), **i32))
    rws = torch.empty(ep.rank_layout_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    y = to_dev(W.gen_y(w), torch.bfloat16)
    part = torch.empty((w.nrows, w.H), dtype=torch.bfloat16, device="cuda")
    out_rk = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")

    def run():
        ep.route(cfg, lg, idx, wt)
        ep.dispatch_ll(cfg, x, idx, cap, "fp8", ll["recv"], ll["scales"], ll["count"], ll["src"], ll["slot"])
        ep.combine_ll(cfg, cap, yll, ll["slot"], wt, out_ll)
        ep.get_layout(cfg, idx, lay, ws, with_recv_token=False)
        ep.get_rank_layout(cfg, idx, rl, rws, with_rank_token=False)
        ep.combine_rank_partial(cfg, y, idx, lay["slot"], wt, rl["rank_slot"], part)
        ep.combine_ranks(cfg, part, rl["rank_slot"], out_rk)

    # rows no pair takes are not written by the calls: leave them out of the
    # comparison (the eager writes between replays would change them)
    outs = [idx, wt, ll["count"], ll["slot"], out_ll, *lay.values(), *rl.values(), out_rk]
    _capture_and_check(run, outs)


def test_fused_route_layout_step_in_graph():
    # the step as the benchmark runs it: ep_route_layout (two launches at
    # this size), FP8 dispatch, combine
    w = W.PREFILL.replace(T=2048)
    cfg = ep.Config.of(w)
    lg = to_dev(W.gen_logits(w))
    x = to_dev(W.gen_x(w), torch.bfloat16)
    y = to_dev(W.gen_y(w), torch.bfloat16)
    i32 = dict(dtype=torch.int32, device="cuda")
    o = dict(idx=torch.empty((w.T, w.k), **i32), w=torch.empty((w.T, w.k), dtype=torch.float32, device="cuda"),
             cnt=torch.empty(w.E, **i32), ntok_rank=torch.empty(w.R, **i32), off=torch.empty(w.E + 1, **i32),
             slot=torch.empty((w.T, w.k), **i32), recv_token=torch.empty(w.nrows, **i32))
    ws = torch.empty(ep.route_layout_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    recv = torch.empty((w.nrows, w.H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((w.nrows, w.H // 128), dtype=torch.float32, device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")

    def run():
        ep.route_layout(cfg, lg, o, ws)
        ep.dispatch(cfg, x, o["slot"], "fp8", recv, sc)
        ep.combine(cfg, y, o["slot"], o["w"], out)

    _capture_and_check(run, [*o.values(), recv, sc, out])
