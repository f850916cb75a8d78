"""ep_route_layout (routing followed by the layout, in two launches where the
routing kernel also counts its picks per 16-token column) against the
oracle's route and layout, bit for bit, and against the separate ep_route
and ep_get_layout calls. Shapes: every workload; random shapes of the pair
gate (E in {128, 256, 512, 1024}, groups of whole lanes or every group kept,
m <= 2, k up to 32, any R) at token counts around the 16-token columns and
the 64-token assign blocks, with normal and tie-heavy logits; the assign
launch's lane strides; the routing launch's two ways of counting
(per-wavefront rows, LDS atomics) at their edges; one and two tokens per
wavefront around 4096 tokens (top-6 keeps the switch, top-8 of 8 groups
stays at one); and shapes that take the fallback path (among them E = 512
and 1024, whose assign launch would need more than 64 KiB of LDS, and E with
a count of experts per lane that is not a power of two: 160, 192, 320, 384,
640 and 768); exact score ties for the pick rounds of 256 experts, four per
lane; logits only 4-byte aligned; and NaN logits (outside the contract: k
distinct experts in range per token, the other tokens as the oracle routes
them)."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu

KEYS = ("cnt", "off", "ntok_rank", "slot", "recv_token")


def say(*a):
    print(*a, flush=True)


def check(w, lg, with_recv_token=True):
    cfg = ep.Config.of(w)
    d = to_dev(lg)
    got = ep.route_layout(cfg, d, with_recv_token=with_recv_token)
    idx, wt = ep.route(cfg, d)
    lay = ep.get_layout(cfg, idx)
    torch.cuda.synchronize()
    oi, ow = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    ol = oracle.layout(oi, w.E, w.R)
    assert np.array_equal(to_host(got["idx"]), oi), "idx"
    assert np.array_equal(to_host(got["w"]).view(np.uint32), ow.view(np.uint32)), "w"
    assert np.array_equal(to_host(idx), oi), "ep_route idx"
    assert np.array_equal(to_host(wt).view(np.uint32), ow.view(np.uint32)), "ep_route w"
    for key in KEYS:
        if key == "recv_token" and not with_recv_token:
            continue
        assert np.array_equal(to_host(got[key]), ol[key]), key
        assert np.array_equal(to_host(lay[key]), ol[key]), "ep_get_layout " + key


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "skewed_literal", "large"])
def test_route_layout_workloads(name):
    w = W.CONFIGS[name]
    say("route_layout", name, w)
    check(w, W.gen_logits(w))


def test_two_launch_path_is_taken_at_prefill():
    # the workspace is the routing step's column histograms: one byte per
    # expert and per rank for each of the 256 columns of 16 tokens
    cfg = ep.Config.of(W.PREFILL)
    C = W.PREFILL.T // 16
    want = -(-C * cfg.E // 256) * 256 + -(-C * cfg.R // 256) * 256
    assert ep.route_layout_workspace_bytes(cfg) == want


def _pair_shape(rng):
    E = int(rng.choice([128, 256, 512, 1024]))
    if rng.random() < 0.25:
        # every group kept: any G dividing E
        G = int(rng.choice([g for g in (1, 2, 3, 4, 8, 16, 32, 64) if E % g == 0]))
        TG, m = G, int(rng.choice([0, 1, 2]))
    else:
        G = int(rng.choice([1, 2, 4, 8, 16, 32]))  # groups of 32/G whole lanes
        TG, m = int(rng.integers(1, G + 1)), int(rng.choice([0, 1, 2]))
    GS = E // G
    k = int(rng.integers(1, min(32, TG * GS) + 1))
    if m == 0 and max(1, k // TG) > 2:
        m = 2
    m = min(m, GS)
    R = int(rng.choice([r for r in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512) if E % r == 0]))
    if rng.random() < 0.7:   # above 1024 pairs: the two-launch path where the shape allows it
        T = int(rng.choice([129, 255, 257, 1000, 1023, 2049, 4095, 4096]))
    else:
        T = int(rng.choice([1, 15, 16, 17, 63, 64, 65, 127]))
    return W.Workload("pair", T=T, H=128, E=E, G=G, TG=TG, k=k, R=R, m=m, seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("case", range(32))
def test_route_layout_random_pair_shapes(case):
    rng = np.random.default_rng(7000 + case)
    w = _pair_shape(rng)
    mode = ("normal", "exact", "ulps")[case % 3]
    say("route_layout random", case, mode, w)
    if mode == "normal":
        lg = W.gen_logits(w)
    else:
        vals = np.float32([-3.0, -0.5, 0.0, 0.75, 2.0])
        lg = rng.choice(vals[: int(rng.integers(1, 6))], size=(w.T, w.E)).astype(np.float32)
        if mode == "ulps":
            steps = rng.integers(0, 3, size=(w.T, w.E)).astype(np.int32)
            lg = (lg.view(np.int32) + np.where(lg >= 0, steps, -steps)).view(np.float32)
    check(w, lg, with_recv_token=bool(case % 4))


def _two_launch(w) -> bool:
    cfg = ep.Config.of(w)
    C = -(-w.T // 16)
    return ep.route_layout_workspace_bytes(cfg) == -(-C * w.E // 256) * 256 + -(-C * w.R // 256) * 256 \
        and w.T * w.k > 1024


@pytest.mark.parametrize("T,k", [(33, 32), (47, 24), (63, 17), (65, 32), (129, 8), (4095, 8), (4096, 8)])
def test_route_layout_column_and_block_edges(T, k):
    # token counts around the 16-token columns and 64-token assign blocks,
    # with enough picks to take the two-launch path
    w = W.PREFILL.replace(name="edges", T=T, k=k, TG=8 if k > 8 else 4, m=2, seed=T * 100 + k)
    assert _two_launch(w)
    say("route_layout edges", w)
    check(w, W.gen_logits(w))


@pytest.mark.parametrize("w", [
    W.Workload("fb_e96", T=333, H=128, E=96, G=4, TG=2, k=6, R=12, m=3, seed=41),     # general gate
    W.Workload("fb_m4", T=200, H=128, E=256, G=8, TG=4, k=16, R=32, m=4, seed=42),    # m > 2
    W.Workload("fb_r1024", T=70, H=128, E=1024, G=8, TG=2, k=8, R=1024, seed=43),     # ranks beyond one block
    W.Workload("fb_e64", T=90, H=128, E=64, G=4, TG=2, k=4, R=8, seed=44),            # E < 128
])
def test_route_layout_fallback_shapes(w):
    say("route_layout fallback", w)
    check(w, W.gen_logits(w))


@pytest.mark.parametrize("w", [
    W.Workload("epl6", T=700, H=128, E=384, G=16, TG=8, k=8, R=48, m=2, seed=51),      # 6 per lane
    W.Workload("epl5", T=500, H=128, E=320, G=64, TG=16, k=8, R=40, m=2, seed=52),     # 5 per lane
    W.Workload("epl10", T=300, H=128, E=640, G=64, TG=8, k=8, R=64, m=2, seed=53),     # 10 per lane
    W.Workload("epl12", T=200, H=128, E=768, G=8, TG=8, k=8, R=96, m=1, seed=54),      # 12, all groups
    W.Workload("epl6h", T=5000, H=128, E=192, G=8, TG=4, k=6, R=24, m=2, seed=55),     # 6 per half-wave lane
    W.Workload("epl5h", T=4500, H=128, E=160, G=5, TG=5, k=6, R=20, m=0, seed=56),     # 5, all groups
], ids=lambda w: w.name)
def test_route_layout_experts_per_lane_not_a_power_of_two(w):
    # E a multiple of the token's lanes, but E / lanes not 4, 8, 16 or 32:
    # the routing kernel that holds runs of experts per lane has no such
    # instance, so these shapes take the other gate kernels
    say("route_layout experts per lane", w)
    check(w, W.gen_logits(w), with_recv_token=w.T % 2 == 0)


def test_route_layout_zero_tokens():
    w = W.PREFILL.replace(T=0)
    cfg = ep.Config.of(w)
    got = ep.route_layout(cfg, torch.empty((0, w.E), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert to_host(got["cnt"]).sum() == 0 and to_host(got["off"]).tolist() == [0] * (w.E + 1)
    assert to_host(got["ntok_rank"]).sum() == 0


@pytest.mark.parametrize("E,G", [(128, 8), (128, 4), (256, 8), (256, 16)])
def test_route_layout_column_reduction_strides(E, G):
    # the assign launch sums each wavefront's row groups with lane strides
    # E/16 = 8 (DPP row rotations, then row swaps) and 16 (row swaps only);
    # E = 128 takes two tokens per wavefront in the routing launch, 256 one
    w = W.Workload("strides", T=1000, H=128, E=E, G=G, TG=G // 2, k=8, R=32, m=2, seed=E + G)
    assert _two_launch(w)
    say("route_layout strides", w)
    check(w, W.gen_logits(w))


@pytest.mark.parametrize("E,G,R,T", [
    (128, 8, 64, 4095), (128, 4, 32, 1023), (128, 8, 128, 2049), (128, 8, 1, 129),
    (256, 8, 64, 4081), (256, 8, 128, 1031), (256, 16, 2, 200),
])
def test_route_layout_count_rows_and_atomics(E, G, R, T):
    # the routing launch counts its picks per column in per-wavefront rows
    # when each lane holds four experts and R <= 64, else with LDS atomics:
    # odd T at 128 experts leaves the last wavefront's upper half without a
    # token, and T off a multiple of 16 leaves tokenless wavefronts in the
    # last column
    w = W.Workload("rows", T=T, H=128, E=E, G=G, TG=G // 2, k=8, R=R, m=2, seed=E * 7 + R + T)
    assert _two_launch(w)
    say("route_layout count rows", w)
    check(w, W.gen_logits(w), with_recv_token=True)


@pytest.mark.parametrize("T,k", [(4095, 8), (4096, 8), (4097, 8), (6000, 8), (4096, 6), (4097, 6), (6000, 6)])
def test_route_one_and_two_tokens_per_wavefront(T, k):
    # the gate takes one token per wavefront up to 4096 tokens and two above,
    # except for the sorted-key rounds (256 experts, top-8 of 8 groups),
    # which keep one token per wavefront at every size
    w = W.PREFILL.replace(name="tpw", T=T, H=128, k=k, seed=T + k)
    say("route tokens per wavefront", w)
    check(w, W.gen_logits(w), with_recv_token=T % 2 == 0)


@pytest.mark.parametrize("w", [W.DECODE, W.PREFILL.replace(T=1024), W.PREFILL.replace(T=6000)],
                         ids=["decode", "prefill_1024", "prefill_6000"])
def test_logits_only_four_byte_aligned(w):
    # the routing kernel reads each lane's logits 16 bytes at a time; the ABI
    # promises 4-byte alignment, so a row start may sit 4 bytes past a
    # 16-byte boundary (one, two-launch and two-tokens-per-wavefront paths)
    say("route_layout, logits at a 4-byte offset", w)
    lg = W.gen_logits(w)
    cfg = ep.Config.of(w)
    buf = torch.zeros(lg.size + 1, dtype=torch.float32, device="cuda")
    buf[1:] = to_dev(lg).view(-1)
    d = buf[1:].view(w.T, w.E)
    assert d.data_ptr() % 16 == 4
    got = ep.route_layout(cfg, d)
    idx, wt = ep.route(cfg, d)
    torch.cuda.synchronize()
    oi, ow = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    ol = oracle.layout(oi, w.E, w.R)
    for name, (gi, gw) in (("route_layout", (got["idx"], got["w"])), ("route", (idx, wt))):
        assert np.array_equal(to_host(gi), oi), name + " idx"
        assert np.array_equal(to_host(gw).view(np.uint32), ow.view(np.uint32)), name + " w"
    for key in KEYS:
        assert np.array_equal(to_host(got[key]), ol[key]), key


@pytest.mark.parametrize("case", range(16))
def test_sorted_key_rounds_with_exact_ties(case):
    # four experts per lane (256 experts at one token per wavefront, 128 at
    # two): the pick rounds read each lane's sorted keys, whose low bits hold
    # the expert's place in the lane; exact score ties within a lane and
    # across lanes must still go to the lower expert index.  Logits from one
    # to four distinct values (exactly equal, or 1-2 ulps apart), group limit
    # on and off, with and without the pick counts; top-8 of 8 groups (picks
    # unrolled) and top-6 or 16 groups (picks counted at run time).
    rng = np.random.default_rng(9100 + case)
    E = 256 if case < 8 or case % 2 else 128
    G, k = (8, 8) if case < 12 else (16, 6)
    TG = G if case % 4 == 0 else G // 2
    T = (77, 1000, 3000, 4096)[case % 4]
    w = W.PREFILL.replace(name="ties%d" % E, T=T, H=128, E=E, G=G, TG=TG, k=k, R=16,
                          m=1 if TG == G else 2, seed=9100 + case)
    vals = np.float32([-1.5, 0.0, 0.25, 3.0])
    lg = rng.choice(vals[: 1 + case % 4], size=(w.T, w.E)).astype(np.float32)
    if case % 2:
        steps = rng.integers(0, 3, size=(w.T, w.E)).astype(np.int32)
        lg = (lg.view(np.int32) + np.where(lg >= 0, steps, -steps)).view(np.float32)
    say("sorted-key rounds, ties", case, w)
    check(w, lg, with_recv_token=bool(case % 2))


@pytest.mark.parametrize("w", [
    W.PREFILL.replace(name="nan256", T=1000, H=128, seed=71),                       # sorted-key rounds
    W.DECODE.replace(name="nan_decode", H=128, seed=72),                            # every group kept
    W.Workload("nan128", T=600, H=128, E=128, G=8, TG=4, k=8, R=16, seed=73),       # lanes of 4, G=8
    W.Workload("nan_e96", T=300, H=128, E=96, G=4, TG=2, k=6, R=12, m=3, seed=74),  # general gate
], ids=["e256", "decode", "e128", "e96"])
def test_nan_logits_still_give_distinct_picks(w):
    # NaN logits are outside the contract (the selection is unspecified), but
    # every token must still get k distinct experts in range, and tokens
    # without a NaN are routed exactly as the oracle routes them
    rng = np.random.default_rng(w.seed)
    lg = W.gen_logits(w)
    bad = rng.random(w.T) < 0.3
    for t in np.flatnonzero(bad):
        lg[t, rng.choice(w.E, size=int(rng.integers(1, w.E + 1)), replace=False)] = np.nan
    say("NaN logits", w, int(bad.sum()), "tokens with NaN")
    cfg = ep.Config.of(w)
    d = to_dev(lg)
    got = ep.route_layout(cfg, d)
    idx, _ = ep.route(cfg, d)
    torch.cuda.synchronize()
    ok = ~bad
    oi, ow = oracle.route(np.ascontiguousarray(lg[ok]), w.G, w.TG, w.k, w.topm)
    for name, gi in (("route_layout", to_host(got["idx"])), ("route", to_host(idx))):
        assert ((gi >= 0) & (gi < w.E)).all(), name
        assert all(len(set(row)) == w.k for row in gi.tolist()), name + ": repeated expert"
        assert np.array_equal(gi[ok], oi), name + ": tokens without NaN"
    assert np.array_equal(to_host(got["w"])[ok].view(np.uint32), ow.view(np.uint32))


def test_layout_calls_return_the_workspace_they_allocate():
    # a workspace the call allocates comes back with its outputs (so that it
    # lives as long as they do, also for work on another stream); one the
    # caller passes does not
    w = W.PREFILL.replace(name="ws", T=300, seed=5)
    cfg = ep.Config.of(w)
    d = to_dev(W.gen_logits(w))
    calls = (
        (lambda ws=None: ep.route_layout(cfg, d, workspace=ws), ep.route_layout_workspace_bytes(cfg)),
        (lambda ws=None: ep.get_layout(cfg, ep.route(cfg, d)[0], workspace=ws), ep.layout_workspace_bytes(cfg)),
        (lambda ws=None: ep.get_rank_layout(cfg, ep.route(cfg, d)[0], workspace=ws),
         ep.rank_layout_workspace_bytes(cfg)),
    )
    for call, need in calls:
        got = call()
        assert got["workspace"].dtype == torch.uint8 and got["workspace"].numel() >= need
        mine = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        assert "workspace" not in call(mine)
    torch.cuda.synchronize()
