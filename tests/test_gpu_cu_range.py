"""The library's calls on streams confined to a range of compute units
(ep_stream_create_cu_range, the CU-budget analogue of the pages' SM-count
control) against the CPU oracle: the normal path (route, layout, the
routing with its layout in two launches, FP8 dispatch, combine), the
low-latency path (dispatch_ll, combine_ll) and the
deduplicated path (rank layout, dispatch over rank slots, in-rank partial
combine, combine of partials), bit for bit (flat combines within 1 bf16
ulp).  Every device input is created before the calls and kept until the
stream has been synchronised; the layout calls' own workspaces come back
with their outputs and are kept as long."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from checks import bf16_ulp_diff
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu

SENT_Q, SENT_SC, NAN_BF16 = 0x5A, -7.0, 0x7FC0


def say(*a):
    print(*a, flush=True)


def same(name, got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    assert got.shape == ref.shape and bad.size == 0, "%s: %d differ" % (name, bad.size)


def within_ulp(name, got, ref):
    d = bf16_ulp_diff(got, ref)
    say("%s: %d of %d elements differ, max %d ulp" % (name, (d > 0).sum(), d.size, d.max()))
    assert d.max() <= 1


def expected(w, lg, x, y, cap):
    """Every output of the three paths, from the oracle alone."""
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    lay = oracle.layout(idx, w.E, w.R)
    e = dict(idx=idx, wt=wt, **lay)
    e["recv"], e["sc"] = oracle.dispatch_fp8(x, lay["slot"], w.nrows)
    e["out"] = oracle.combine(y, lay["slot"], wt)
    ll = oracle.ll_layout(idx, w.E, cap)
    nll = w.E * cap
    e["ll_slot"], e["ll_count"] = ll["slot"], ll["count"]
    e["ll_recv"], e["ll_sc"] = oracle.dispatch_fp8(x, ll["slot"], nll, np.full((nll, w.H), SENT_Q, np.uint8),
                                                   np.full((nll, w.H // 128), SENT_SC, np.float32))
    # low-latency expert outputs: y's rows where a pair landed, NaN elsewhere
    yll = np.full((nll, w.H), NAN_BF16, np.uint16)
    taken = np.sort(ll["slot"][ll["slot"] >= 0])
    yll[taken] = y[: taken.size]
    e["ll_y"] = yll
    e["ll_out"] = oracle.combine(yll, ll["slot"], wt)
    rl = oracle.rank_layout(idx, w.E, w.R)
    e.update(rl)
    e["rk_recv"], e["rk_sc"] = oracle.dispatch_fp8(x, rl["rank_slot"], w.nrows,
                                                   np.full((w.nrows, w.H), SENT_Q, np.uint8),
                                                   np.full((w.nrows, w.H // 128), SENT_SC, np.float32))
    e["part"] = oracle.combine_rank_partial(y, idx, lay["slot"], wt, rl["rank_slot"], w.E, w.R, w.nrows,
                                            np.zeros((w.nrows, w.H), np.uint16))
    e["rk_out"] = oracle.combine_ranks(e["part"], rl["rank_slot"])
    return e


def run_on(stream, w, cfg, d, cap):
    """All three paths on `stream`; returns host copies of every output."""
    idx, wt = ep.route(cfg, d["lg"], stream=stream)
    lay = ep.get_layout(cfg, idx, stream=stream)
    fused = ep.route_layout(cfg, d["lg"], stream=stream)
    recv, sc = ep.dispatch(cfg, d["x"], lay["slot"], stream=stream)
    out = ep.combine(cfg, d["y"], lay["slot"], wt, stream=stream)
    nll = w.E * cap
    ll_recv = torch.full((nll, w.H), SENT_Q, dtype=torch.uint8, device="cuda")
    ll_sc = torch.full((nll, w.H // 128), SENT_SC, dtype=torch.float32, device="cuda")
    ll = ep.dispatch_ll(cfg, d["x"], idx, cap, "fp8", ll_recv, ll_sc, stream=stream)
    ll_out = ep.combine_ll(cfg, cap, d["yll"], ll["slot"], wt, stream=stream)
    rl = ep.get_rank_layout(cfg, idx, stream=stream)
    rk_recv = torch.full((w.nrows, w.H), SENT_Q, dtype=torch.uint8, device="cuda")
    rk_sc = torch.full((w.nrows, w.H // 128), SENT_SC, dtype=torch.float32, device="cuda")
    ep.dispatch(cfg, d["x"], rl["rank_slot"], "fp8", rk_recv, rk_sc, stream=stream)
    part = torch.zeros((w.nrows, w.H), dtype=torch.bfloat16, device="cuda")
    ep.combine_rank_partial(cfg, d["y"], idx, lay["slot"], wt, rl["rank_slot"], part, stream=stream)
    rk_out = ep.combine_ranks(cfg, part, rl["rank_slot"], stream=stream)
    torch.cuda.synchronize()
    g = dict(idx=idx, wt=wt, recv=recv, sc=sc, out=out, ll_slot=ll["slot"], ll_count=ll["count"],
             ll_recv=ll_recv, ll_sc=ll_sc, ll_out=ll_out, rk_recv=rk_recv, rk_sc=rk_sc, part=part, rk_out=rk_out)
    g.update({k: v for k, v in lay.items() if k != "workspace"})
    g.update({k: v for k, v in rl.items() if k != "workspace"})
    g.update({"fused_" + k: v for k, v in fused.items() if k != "workspace"})
    return {k: to_host(v) for k, v in g.items()}


def test_cu_range_streams_match_oracle():
    w = W.PREFILL.replace(T=512)
    cap = 20   # below the largest expert count at 512 tokens (mean 16): some pairs are dropped
    say("cu-range streams", w, "capacity", cap)
    lg, x, y = W.gen_logits(w), W.gen_x(w), W.gen_y(w)
    e = expected(w, lg, x, y, cap)
    assert (e["ll_slot"] < 0).any()
    cfg = ep.Config.of(w)
    # device inputs, alive until after every synchronisation below
    d = dict(lg=to_dev(lg), x=to_dev(x, torch.bfloat16), y=to_dev(y, torch.bfloat16),
             yll=to_dev(e["ll_y"], torch.bfloat16))
    torch.cuda.synchronize()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    for first, num in ((0, 24), (0, 32), (ncu // 2, ncu // 2)):
        say("CUs [%d, %d)" % (first, first + num))
        with ep.CuRangeStream(first, num) as s:
            g = run_on(s, w, cfg, d, cap)
        for key in ("idx", "wt", "cnt", "off", "ntok_rank", "slot", "recv_token", "recv", "sc",
                    "ll_slot", "ll_count", "ll_recv", "ll_sc", "rank_count", "rank_offset", "rank_slot",
                    "rank_token", "rk_recv", "rk_sc", "part", "rk_out"):
            same(key, g[key], e[key])
        for key in ("cnt", "off", "ntok_rank", "slot", "recv_token"):
            same("route_layout " + key, g["fused_" + key], e[key])
        same("route_layout idx", g["fused_idx"], e["idx"])
        same("route_layout w", g["fused_w"], e["wt"])
        within_ulp("combine", g["out"], e["out"])
        within_ulp("combine_ll", g["ll_out"], e["ll_out"])
