"""Parity over seeded random valid configurations: every call (route,
layout, FP8 and BF16 dispatch, combine, low-latency dispatch and combine,
rank layout, partial combine, combine of partials) against the oracle on
shapes drawn from the documented limits, so that every kernel branch (gate
fast/general paths, two- and three-launch layouts, k batches) meets
unusual sizes."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from checks import bf16_ulp_diff
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu


def _draw(rng):
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    GS = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 32, 64]))
    while G * GS > 1024:
        GS //= 2
    E = G * GS
    divs = [r for r in range(1, E + 1) if E % r == 0]
    R = int(rng.choice(divs))
    TG = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, min(32, TG * GS) + 1))
    m = min(int(rng.choice([0, 0, 1, 2, 8])), GS)
    if m == 0 and max(1, k // TG) > min(GS, 8):
        m = min(GS, 8)
    T = int(rng.choice([1, 5, 63, 64, 65, 130, 257, 600]))
    H = int(rng.choice([128, 256, 384, 640, 1024]))
    return W.Workload("sweep", T=T, H=H, E=E, G=G, TG=TG, k=k, R=R, m=m, seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("case", range(24))
def test_random_config(case):
    rng = np.random.default_rng(1000 + case)
    w = _draw(rng)
    cfg = ep.Config.of(w)
    ep.validate(cfg)
    print("sweep", case, w, flush=True)
    lg, x, y = W.gen_logits(w), W.gen_x(w), W.gen_y(w)
    d_lg, d_x, d_y = to_dev(lg), to_dev(x, torch.bfloat16), to_dev(y, torch.bfloat16)
    idx, wt = ep.route(cfg, d_lg)
    lay = ep.get_layout(cfg, idx)
    q, s = ep.dispatch(cfg, d_x, lay["slot"], "fp8")
    b16, _ = ep.dispatch(cfg, d_x, lay["slot"], "bf16")
    out = ep.combine(cfg, d_y, lay["slot"], wt)
    rl = ep.get_rank_layout(cfg, idx)
    part = ep.combine_rank_partial(cfg, d_y, idx, lay["slot"], wt, rl["rank_slot"])
    out2 = ep.combine_ranks(cfg, part, rl["rank_slot"])
    torch.cuda.synchronize()

    oi, ow = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    assert np.array_equal(to_host(idx), oi)
    assert np.array_equal(to_host(wt).view(np.uint32), ow.view(np.uint32))
    ol = oracle.layout(oi, w.E, w.R)
    for key in ("cnt", "off", "ntok_rank", "slot", "recv_token"):
        assert np.array_equal(to_host(lay[key]), ol[key]), key
    used = int(ol["off"][-1])
    oq, osc = oracle.dispatch_fp8(x, ol["slot"], w.nrows)
    assert np.array_equal(to_host(q)[:used], oq[:used])
    assert np.array_equal(to_host(s)[:used].view(np.uint32), osc[:used].view(np.uint32))
    assert np.array_equal(to_host(b16)[:used], oracle.dispatch_bf16(x, ol["slot"], w.nrows)[:used])
    assert bf16_ulp_diff(to_host(out), oracle.combine(y, ol["slot"], ow)).max() <= 1
    orl = oracle.rank_layout(oi, w.E, w.R)
    for key in ("rank_count", "rank_offset", "rank_slot", "rank_token"):
        assert np.array_equal(to_host(rl[key]), orl[key]), key
    ru = int(orl["rank_offset"][-1])
    op = oracle.combine_rank_partial(y, oi, ol["slot"], ow, orl["rank_slot"], w.E, w.R, w.nrows)
    assert np.array_equal(to_host(part)[:ru], op[:ru])
    assert np.array_equal(to_host(out2), oracle.combine_ranks(op, orl["rank_slot"]))

    if w.T * w.k <= 8192:
        cap = int(rng.integers(1, w.T + 1))
        ll = ep.dispatch_ll(cfg, d_x, idx, cap, "fp8")
        nr = w.E * cap
        torch.cuda.synchronize()
        oll = oracle.ll_layout(oi, w.E, cap, src=to_host(ll["src"]).copy())
        assert np.array_equal(to_host(ll["count"]), oll["count"])
        assert np.array_equal(to_host(ll["slot"]), oll["slot"])
        assert np.array_equal(to_host(ll["src"]), oll["src"])
        taken = np.sort(oll["slot"][oll["slot"] >= 0])
        lq, ls = oracle.dispatch_fp8(x, oll["slot"], nr)
        assert np.array_equal(to_host(ll["recv"])[taken], lq[taken])
        assert np.array_equal(to_host(ll["scales"])[taken].view(np.uint32), ls[taken].view(np.uint32))
        yll = np.zeros((nr, w.H), np.uint16)
        yll[taken] = W.gen_y(w, nrows=max(1, taken.size))[: taken.size]
        o3 = ep.combine_ll(cfg, cap, to_dev(yll, torch.bfloat16), ll["slot"], wt)
        torch.cuda.synchronize()
        assert bf16_ulp_diff(to_host(o3), oracle.combine(yll, oll["slot"], ow)).max() <= 1


def _tied_logits(rng, T, E, mode):
    # few distinct values, so that scores and group scores tie exactly and
    # the index rules decide; "ulps" adds 0-2 ulp steps, so that nearly
    # equal logits map to equal or adjacent scores
    vals = np.float32([-3.0, -0.5, 0.0, 0.75, 2.0])
    lg = rng.choice(vals[: int(rng.integers(1, 6))], size=(T, E)).astype(np.float32)
    if mode == "ulps":
        steps = rng.integers(0, 3, size=(T, E)).astype(np.int32)
        lg = (lg.view(np.int32) + np.where(lg >= 0, steps, -steps)).view(np.float32)
    return lg


@pytest.mark.parametrize("case", range(16))
def test_random_config_tied_logits(case):
    rng = np.random.default_rng(5000 + case)
    w = _draw(rng)
    mode = "ulps" if case % 2 else "exact"
    cfg = ep.Config.of(w)
    print("tied sweep", case, mode, w, flush=True)
    lg = _tied_logits(rng, w.T, w.E, mode)
    idx, wt = ep.route(cfg, to_dev(lg))
    lay = ep.get_layout(cfg, idx)
    rl = ep.get_rank_layout(cfg, idx)
    torch.cuda.synchronize()
    oi, ow = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    assert np.array_equal(to_host(idx), oi)
    assert np.array_equal(to_host(wt).view(np.uint32), ow.view(np.uint32))
    ol = oracle.layout(oi, w.E, w.R)
    for key in ("cnt", "off", "ntok_rank", "slot", "recv_token"):
        assert np.array_equal(to_host(lay[key]), ol[key]), key
    orl = oracle.rank_layout(oi, w.E, w.R)
    for key in ("rank_count", "rank_offset", "rank_slot", "rank_token"):
        assert np.array_equal(to_host(rl[key]), orl[key]), key
