"""Pins for the oracle's group-limited top-k gating.

Checked against hand-worked cases, against a brute-force enumeration of
every candidate group set and expert set (a different algorithm from the
oracle's repeated best-of search), and against plain top-k where the group
limit does not bind (TG = G, or G = 1)."""
import itertools

import numpy as np
import pytest

import oracle
import workloads as W
from checks import golden_lines


def _key(s):
    """Sort key of the ranking order: score bits descending, index ascending."""
    return lambda i: (-int(np.float32(s[i]).view(np.uint32)), i)


def test_golden_worked_examples():
    n = 0
    for line in golden_lines("gating_cases.txt"):
        head, sc, idx, w = [p.split() for p in line.split("|")]
        E, G, TG, k, m = map(int, head)
        s = np.float32([float(v) for v in sc]).reshape(1, E)
        got_idx, got_w = oracle.select(s, G, TG, k, m)
        assert got_idx[0].tolist() == [int(v) for v in idx], line
        assert np.array_equal(got_w[0], np.float32([float(v) for v in w])), line
        n += 1
    assert n >= 5


def _brute_force(s, G, TG, k, m):
    E = s.shape[0]
    GS = E // G
    gsc = []
    for g in range(G):
        vals = sorted(s[g * GS:(g + 1) * GS].tolist(), key=lambda v: -int(np.float32(v).view(np.uint32)))
        acc = np.float32(0)
        for v in vals[:m]:
            acc = np.float32(acc + np.float32(v))
        gsc.append(acc)
    gk = _key(np.float32(gsc))
    # the kept set is the unique TG-subset whose every member outranks every
    # non-member
    kept = [c for c in itertools.combinations(range(G), TG)
            if all(gk(a) < gk(b) for a in c for b in range(G) if b not in c)]
    assert len(kept) == 1
    cand = [e for e in range(E) if e // GS in kept[0]]
    ek = _key(s)
    chosen = [c for c in itertools.combinations(cand, k)
              if all(ek(a) < ek(b) for a in c for b in cand if b not in c)]
    assert len(chosen) == 1
    return sorted(chosen[0], key=ek)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("m", [1, 2])
def test_brute_force_tiny(seed, m):
    rng = np.random.default_rng(seed)
    T, E, G, TG, k = 64, 16, 4, 2, 4
    # scores on a coarse grid so that exact ties (scores and group scores)
    # are frequent and the tie rules are exercised
    s = (rng.integers(0, 9, size=(T, E)) / 8.0).astype(np.float32)
    idx, w = oracle.select(s, G, TG, k, m)
    for t in range(T):
        assert idx[t].tolist() == _brute_force(s[t], G, TG, k, m), t


def test_brute_force_on_sigmoid_scores():
    w = W.TINY
    s = oracle.scores(W.gen_logits(w))
    idx, _ = oracle.select(s, w.G, w.TG, w.k, w.topm)
    for t in range(w.T):
        assert idx[t].tolist() == _brute_force(s[t], w.G, w.TG, w.k, w.topm)


def _plain_topk(s, k):
    E = s.shape[1]
    bits = s.view(np.uint32).astype(np.int64)
    order = np.lexsort((np.broadcast_to(np.arange(E), s.shape), -bits), axis=1)
    return order[:, :k]


@pytest.mark.parametrize("G", [1, 8])
def test_no_group_limit_is_plain_topk(G):
    rng = np.random.default_rng(3)
    s = oracle.scores(rng.standard_normal((256, 256), dtype=np.float32))
    s[:, 17] = s[:, 18]          # force ties at the selection boundary
    idx, _ = oracle.select(s, G, G, 8, 1)
    assert np.array_equal(idx, _plain_topk(s, 8))


def test_decode_config_equals_plain_topk():
    w = W.DECODE
    assert w.TG == w.G
    lg = W.gen_logits(w)
    idx, _ = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    assert np.array_equal(idx, _plain_topk(oracle.scores(lg), w.k))


def test_weights_closed_form():
    w = W.PREFILL.replace(T=512)
    lg = W.gen_logits(w)
    s = oracle.scores(lg)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    sel = np.take_along_axis(s, idx, axis=1).astype(np.float64)
    # sum to one within the rounding of k quotients and a k-term sum
    assert np.all(np.abs(wt.astype(np.float64).sum(1) - 1.0) <= 2 * w.k * 2.0 ** -24)
    # proportional to the selected scores
    ref = sel / sel.sum(1, keepdims=True)
    assert np.all(np.abs(wt - ref) <= (w.k + 1) * 2.0 ** -24 * ref + 1e-30)
    # picks are distinct, in-range, non-increasing in score, within kept groups
    assert np.all(np.diff(sel, axis=1) <= 0)
    for t in range(w.T):
        assert len(set(idx[t].tolist())) == w.k
        assert len(set((idx[t] // (w.E // w.G)).tolist())) <= w.TG


def test_route_is_select_of_scores():
    w = W.SKEWED.replace(T=256)
    lg = W.gen_logits(w)
    a = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    b = oracle.select(oracle.scores(lg), w.G, w.TG, w.k, w.topm)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_group_limit_changes_the_answer():
    # a check that the limit is applied at all: for prefill-like scores the
    # group-limited pick differs from plain top-8 on many tokens
    w = W.PREFILL.replace(T=512)
    s = oracle.scores(W.gen_logits(w))
    idx, _ = oracle.select(s, w.G, w.TG, w.k, w.topm)
    plain = _plain_topk(s, w.k)
    assert (idx != plain).any(axis=1).mean() > 0.2


@pytest.mark.parametrize("args", [(4, 5, 2, 1), (4, 2, 9, 1), (4, 2, 2, 5), (3, 2, 2, 1), (4, 0, 2, 1)])
def test_invalid_configs_rejected(args):
    G, TG, k, m = args
    s = np.zeros((2, 16), np.float32)
    with pytest.raises(ValueError):
        oracle.select(s, G, TG, k, m)
