"""ep_scores against the oracle's sigmoid, bit for bit: a dense sweep of
fp32 logits over [-100, 100] (every binade, both saturation regions, every
pattern near the cut-offs of the exponential) and special values, on the four-wide and the
scalar kernel path, in place and out of place; and the scores ep_route
ranks: its weights are the chosen scores over their ordered sum."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def sweep_values():
    # every 61st fp32 bit pattern from +0 to 100.0, both signs, and the
    # exponential's cut-offs with their neighbours
    pos = np.arange(0, 0x42C80001, 61, dtype=np.uint32).view(np.float32)
    edges = np.float32([88.72283935546875, -88.72283935546875, -87.33654022216797, 87.33654022216797,
                        88.0, -88.0, 0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 17.0, -17.0, 104.0, -104.0])
    near = np.concatenate([np.nextafter(edges[:6], np.float32(np.inf)), np.nextafter(edges[:6], np.float32(-np.inf))])
    # every fp32 pattern within 4096 of the exponential's range ends (logit
    # -x reaches them), where the two-factor scaling and the subnormal
    # sigmoid results are
    u = np.concatenate([np.arange(b - 4096, b + 4096, dtype=np.uint32) for b in (0x42B17218, 0x42AEAC4F)])
    dense = u.view(np.float32)
    return np.concatenate([pos, -pos, edges, near.astype(np.float32), dense, -dense])


def check(got, ref, name):
    g, r = got.view(np.uint32).ravel(), ref.view(np.uint32).ravel()
    bad = np.flatnonzero(g != r)
    assert bad.size == 0, "%s: %d of %d differ, first at flat index %d: got %r want %r" % (
        name, bad.size, g.size, bad[0], got.ravel()[bad[0]], ref.ravel()[bad[0]])


def test_scores_sweep_bit_exact():
    v = sweep_values()
    E = 1024
    T = -(-v.size // E)
    lg = np.zeros(T * E, np.float32)
    lg[:v.size] = v
    lg = lg.reshape(T, E)
    cfg = ep.Config(T=T, H=128, E=E, G=64, TG=1, k=1, R=1)
    say("scores sweep", T, "x", E)
    ref = oracle.scores(lg)
    got = to_host(ep.scores(cfg, to_dev(lg)))
    check(got, ref, "four-wide path")
    # scalar path: both pointers 4-byte but not 16-byte aligned
    buf = torch.empty(T * E + 1, dtype=torch.float32, device="cuda")
    buf[1:] = to_dev(lg).view(-1)
    out = torch.empty(T * E + 1, dtype=torch.float32, device="cuda")
    ep.scores(cfg, buf[1:].view(T, E), out[1:].view(T, E))
    check(to_host(out[1:]).reshape(T, E), ref, "scalar path")
    # in place
    x = to_dev(lg)
    ep.scores(cfg, x, x)
    check(to_host(x), ref, "in place")


@pytest.mark.parametrize("T,E,G", [(1, 8, 1), (7, 99, 1), (333, 96, 4), (3, 1024, 64)])
def test_scores_ragged_shapes(T, E, G):
    cfg = ep.Config(T=T, H=128, E=E, G=G, TG=1, k=1, R=1)
    rng = np.random.default_rng(T * 1000 + E)
    lg = (rng.standard_normal((T, E)) * 6).astype(np.float32)
    guard = torch.full((T * E + 5,), 7.0, dtype=torch.float32, device="cuda")
    ep.scores(cfg, to_dev(lg), guard[:T * E].view(T, E))
    check(to_host(guard[:T * E]).reshape(T, E), oracle.scores(lg), "ragged %dx%d" % (T, E))
    assert torch.all(guard[T * E:] == 7.0)


def test_route_weights_are_the_ranked_scores():
    cfg = ep.Config(T=4096, H=7168, E=256, G=8, TG=4, k=8, R=32)
    rng = np.random.default_rng(7)
    lg = (rng.standard_normal((cfg.T, cfg.E)) * 2).astype(np.float32)
    d = to_dev(lg)
    idx, wt = ep.route(cfg, d)
    s = to_host(ep.scores(cfg, d))
    idx, wt = to_host(idx), to_host(wt)
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)   # best first
    S = np.zeros(cfg.T, np.float32)
    for j in range(cfg.k):
        S = (S + sel[:, j]).astype(np.float32)
    w = (sel / S[:, None]).astype(np.float32)
    check(wt, w, "weights from scores")


def test_short_sigmoid_equals_the_general_form_on_its_whole_domain():
    """Every fp32 value with |x| <= 80 (the domain of the short sigmoid form
    the kernels take when a whole wavefront's logits lie in it) goes through
    both device forms; their bits must agree everywhere.  The general form is
    the one the sweeps above compare with the oracle."""
    import ctypes

    from combine_group_limited_amd import build as B
    lib = ctypes.CDLL(B.CHECK_LIB_PATH)
    lib.ep_check_sigmoid_inrange.argtypes = [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    say("exhaustive short-sigmoid check, |x| <= 80")
    rc = lib.ep_check_sigmoid_inrange(80.0, counts.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    tested, bad = (int(v) for v in counts.cpu())
    assert tested == 2 * (0x42A00000 + 1), tested  # every pattern from -80 to 80, both zeros
    assert bad == 0, "%d inputs differ" % bad
