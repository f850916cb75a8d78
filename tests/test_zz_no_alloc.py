"""ep_get_layout_static (the layout with the library's static device
scratch in place of a workspace argument), called through the C ABI
binding, against ep_get_layout with its own workspace: several calls in a
row on one stream, each smaller than the one before, every output bit for
bit (and against the oracle)."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from combine_group_limited_amd import _lib as L
from pipeline import to_dev, to_host

pytestmark = pytest.mark.gpu

KEYS = ("cnt", "off", "ntok_rank", "slot", "recv_token")


def say(*a):
    print(*a, flush=True)


def routed(w):
    idx, _ = oracle.route(W.gen_logits(w), w.G, w.TG, w.k, w.topm)
    return idx


def random_ids(w, seed):
    # hand-made topk_idx with unrouted (-1, >= E) and repeated entries
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, w.E, size=(w.T, w.k)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    idx[rng.random(idx.shape) < 0.02] = w.E + 7
    return idx


def test_static_scratch_layout_matches_workspace_layout():
    # the largest batch whose scratch fits (256 experts, 32 ranks, top-8),
    # then the large batch (three launches, 256 count blocks), prefill (two
    # launches, 64 count blocks), a ragged 1000-token batch and a batch the
    # one-workgroup kernel takes (no scratch)
    E, R, k = 256, 32, 8
    fits = (L.EP_STATIC_SCRATCH_BYTES // (4 * (E + R))) * 512 // k
    cases = [
        (W.PREFILL.replace(name="max", T=fits), None),
        (W.LARGE, "routed"),
        (W.PREFILL, "routed"),
        (W.PREFILL.replace(name="ragged", T=1000, E=96, G=4, TG=2, k=6, R=12, m=3), None),
        (W.DECODE, "routed"),
    ]
    got = []
    for i, (w, how) in enumerate(cases):
        cfg = ep.Config.of(w)
        assert ep.layout_workspace_bytes(cfg) <= L.EP_STATIC_SCRATCH_BYTES
        idx = routed(w) if how == "routed" else random_ids(w, 100 + i)
        say("static layout", i, w.name, "T=%d" % w.T, "workspace bytes", ep.layout_workspace_bytes(cfg))
        d = to_dev(idx)
        st = ep.get_layout_static(cfg, d)
        ref = ep.get_layout(cfg, d)
        got.append((w, idx, st, ref, d))
    torch.cuda.synchronize()
    for w, idx, st, ref, _ in got:
        ol = oracle.layout(idx, w.E, w.R)
        for key in KEYS:
            a, b = to_host(st[key]), to_host(ref[key])
            assert np.array_equal(a, b), (w.name, key)
            assert np.array_equal(a, ol[key]), (w.name, key, "oracle")
    say("static layout: %d calls bit-identical to ep_get_layout and the oracle" % len(got))


def test_static_scratch_rejects_beyond_its_size():
    w = W.PREFILL.replace(T=(L.EP_STATIC_SCRATCH_BYTES // (4 * 288)) * 64 + 64)
    cfg = ep.Config.of(w)
    assert ep.layout_workspace_bytes(cfg) > L.EP_STATIC_SCRATCH_BYTES
    with pytest.raises(ep.EpError, match="static array"):
        ep.get_layout_static(cfg, torch.zeros((w.T, w.k), dtype=torch.int32, device="cuda"))
