"""Parity of the per-rank deduplicated path (ep_get_rank_layout, ep_dispatch
over rank_slot, ep_combine_rank_partial, ep_combine_ranks, called through
the C ABI binding) with the CPU oracle: bit-exact layout, payload and
scales, partial rows and final rows (both sides run the same fp32 chains
in the same order)."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from checks import bf16_ulp_diff
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_and_check(w, idx, wt, x, y):
    cfg = ep.Config.of(w)
    d_idx, d_wt = to_dev(idx), to_dev(wt)
    lay = ep.get_layout(cfg, d_idx)
    rl = ep.get_rank_layout(cfg, d_idx)
    recv = torch.full((w.nrows, w.H), 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.full((w.nrows, w.H // 128), -7.0, dtype=torch.float32, device="cuda")
    ep.dispatch(cfg, to_dev(x, torch.bfloat16), rl["rank_slot"], "fp8", recv, sc)
    part = torch.full((w.nrows, w.H), 0x1234, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ep.combine_rank_partial(cfg, to_dev(y, torch.bfloat16), d_idx, lay["slot"], d_wt, rl["rank_slot"], part)
    out = ep.combine_ranks(cfg, part, rl["rank_slot"])
    torch.cuda.synchronize()

    ol = oracle.layout(idx, w.E, w.R)
    orl = oracle.rank_layout(idx, w.E, w.R)
    for key in ("rank_count", "rank_offset", "rank_slot", "rank_token"):
        assert np.array_equal(to_host(rl[key]), orl[key]), key
    assert np.array_equal(to_host(lay["slot"]), ol["slot"])
    q, s = oracle.dispatch_fp8(x, orl["rank_slot"], w.nrows, np.full((w.nrows, w.H), 0x5A, np.uint8),
                               np.full((w.nrows, w.H // 128), -7.0, np.float32))
    assert np.array_equal(to_host(recv), q)
    assert np.array_equal(to_host(sc).view(np.uint32), s.view(np.uint32))
    op = oracle.combine_rank_partial(y, idx, ol["slot"], wt, orl["rank_slot"], w.E, w.R, w.nrows,
                                     np.full((w.nrows, w.H), 0x1234, np.uint16))
    assert np.array_equal(to_host(part), op)
    oo = oracle.combine_ranks(op, orl["rank_slot"])
    d = bf16_ulp_diff(to_host(out), oo)
    used = int(orl["rank_offset"][-1])
    say("rank path: %d rank rows for %d pairs (%.2f per token); final rows differ in %d elements" % (
        used, (idx >= 0).sum(), used / max(w.T, 1), (d > 0).sum()))
    assert d.max() == 0


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed"])
def test_rank_path_routed(name):
    # full size: prefill and skewed are the 4096-token batches the
    # deduplicated bench path times
    w = W.CONFIGS[name]
    say("rank path", name, w)
    lg, x, y = W.gen_logits(w), W.gen_x(w), W.gen_y(w)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    run_and_check(w, idx, wt, x, y)


@pytest.mark.parametrize("w", [
    W.Workload("rk_k32", T=150, H=256, E=1024, G=64, TG=8, k=32, R=64, m=4, seed=31),
    W.Workload("rk_k16", T=200, H=512, E=64, G=4, TG=1, k=16, R=2, m=8, seed=32),
    W.Workload("rk_r1", T=99, H=384, E=96, G=4, TG=2, k=6, R=1, m=3, seed=33),
    W.Workload("rk_re", T=64, H=128, E=16, G=4, TG=2, k=4, R=16, seed=34),
])
def test_rank_path_edge_shapes(w):
    say("rank path edge", w)
    lg, x, y = W.gen_logits(w), W.gen_x(w), W.gen_y(w)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    run_and_check(w, idx, wt, x, y)


def test_rank_path_unrouted_and_repeated():
    w = W.Workload("rk_holes", T=400, H=512, E=48, G=4, TG=4, k=6, R=8, seed=35)
    say("rank path holes", w)
    rng = np.random.default_rng(35)
    idx = rng.integers(0, w.E, size=(w.T, w.k)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    idx[rng.random(idx.shape) < 0.03] = w.E + 2
    wt = rng.random((w.T, w.k)).astype(np.float32)
    run_and_check(w, idx, wt, W.gen_x(w), W.gen_y(w))


def test_rank_layout_large_batch():
    # 16384 tokens x top-8 = 131072 picks: the layout over the 32 rank
    # buckets takes the three-launch path (more than 64 count blocks)
    w = W.LARGE
    say("rank layout large", w)
    idx, _ = oracle.route(W.gen_logits(w), w.G, w.TG, w.k, w.topm)
    cfg = ep.Config.of(w)
    rl = ep.get_rank_layout(cfg, to_dev(idx))
    torch.cuda.synchronize()
    orl = oracle.rank_layout(idx, w.E, w.R)
    for key in ("rank_count", "rank_offset", "rank_slot", "rank_token"):
        assert np.array_equal(to_host(rl[key]), orl[key]), key
