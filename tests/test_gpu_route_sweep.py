"""Routing and layout over random shapes drawn from the whole validated space:
any G <= 64, any group size with E <= 1024, top-m up to 8, k up to 32, any R
dividing E, 1 to 5000 tokens. A third of the cases take the shapes of the
routing kernel that holds runs of experts per lane (E of 128 to 1024,
power-of-two groups, top-m <= 2), a third E from a list of sizes around the
kernels' boundaries (multiples of 32 and 64, powers of two or not), a third
any G and group size. So every routing kernel and token packing, and every
layout path, meets shapes chosen without regard to which kernel serves them.
ep_route, ep_get_layout and ep_route_layout are checked against the oracle
bit for bit, with normal and tie-heavy logits."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu

BOUNDARY_E = (64, 96, 128, 160, 192, 256, 320, 384, 448, 512, 640, 768, 896, 1024)
KEYS = ("cnt", "off", "ntok_rank", "slot", "recv_token")


def _shape(rng, case):
    while True:
        kind = case % 3
        if kind == 0:  # the lane-run kernel's shapes: power-of-two groups, top-m <= 2
            E = int(rng.choice([128, 256, 512, 1024]))
            G = int(rng.choice([g for g in (1, 2, 4, 8, 16, 32, 64) if E % g == 0]))
        elif kind == 1:
            E = int(rng.choice(BOUNDARY_E))
            G = int(rng.choice([g for g in range(1, 65) if E % g == 0]))
        else:
            G = int(rng.integers(1, 65))
            E = G * int(rng.integers(1, 1024 // G + 1))
        GS = E // G
        TG = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(32, TG * GS) + 1))
        m = int(rng.choice([0, 1, 2]) if kind == 0 else rng.choice([0, 0, 1, 2, 3, 8]))
        if (m or max(1, k // TG)) > (min(GS, 2) if kind == 0 else min(GS, 8)):
            continue
        R = int(rng.choice([r for r in range(1, E + 1) if E % r == 0]))
        T = int(rng.choice([1, 7, 64, 100, 333, 1000, 2049, 4096, 4097, 5000]))
        return W.Workload("rsweep", T=T, H=128, E=E, G=G, TG=TG, k=k, R=R, m=m, seed=int(rng.integers(1 << 30)))


def _logits(rng, w, mode):
    if mode == "normal":
        return W.gen_logits(w)
    vals = np.float32([-3.0, -0.5, 0.0, 0.75, 2.0])
    return rng.choice(vals[: int(rng.integers(1, 6))], size=(w.T, w.E)).astype(np.float32)


@pytest.mark.parametrize("case", range(48))
def test_route_and_layout_random_shapes(case):
    rng = np.random.default_rng(9100 + case)
    w = _shape(rng, case)
    mode = "ties" if case % 4 == 3 else "normal"
    print("route sweep", case, mode, w, flush=True)
    cfg = ep.Config.of(w)
    ep.validate(cfg)
    lg = _logits(rng, w, mode)
    d = to_dev(lg)
    idx, wt = ep.route(cfg, d)
    lay = ep.get_layout(cfg, idx)
    fused = ep.route_layout(cfg, d)
    torch.cuda.synchronize()
    oi, ow = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    ol = oracle.layout(oi, w.E, w.R)
    for got_i, got_w, where in ((idx, wt, "ep_route"), (fused["idx"], fused["w"], "ep_route_layout")):
        assert np.array_equal(to_host(got_i), oi), where + " idx"
        assert np.array_equal(to_host(got_w).view(np.uint32), ow.view(np.uint32)), where + " w"
    for key in KEYS:
        assert np.array_equal(to_host(lay[key]), ol[key]), "ep_get_layout " + key
        assert np.array_equal(to_host(fused[key]), ol[key]), "ep_route_layout " + key
