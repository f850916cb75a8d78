"""Pins for the oracle's low-latency receive layout (fixed rows per expert):
hand-worked cases, a stable sort of the flattened expert ids (library
routine) giving each pair's arrival position, and the relation to the
canonical layout when nothing overflows."""
import numpy as np
import pytest

import oracle
import workloads as W
from checks import golden_lines


def _ints(s):
    return [int(v) for v in s.split()]


def _golden():
    for line in golden_lines("ll_layout_cases.txt"):
        head, idx, count, slot, src = [p.strip() for p in line.split("|")]
        E, cap = _ints(head)
        rows = [_ints(r) for r in idx.split(";")]
        srows = [_ints(r) for r in slot.split(";")]
        yield E, cap, np.array(rows, np.int32), _ints(count), np.array(srows, np.int32), src.split()


@pytest.mark.parametrize("case", list(_golden()))
def test_hand_worked_cases(case):
    E, cap, idx, count, slot, src = case
    L = oracle.ll_layout(idx, E, cap, src=np.full(E * cap, -99, np.int32))
    assert L["count"].tolist() == count
    assert np.array_equal(L["slot"], slot)
    for row, v in enumerate(src):
        assert L["src"][row] == (-99 if v == "x" else int(v))


def _expected_by_sort(idx, E, cap):
    T, k = idx.shape
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")            # pairs grouped by expert, arrival order kept
    sorted_e = key[order]
    first = np.searchsorted(sorted_e, sorted_e, side="left")
    pos = np.empty(T * k, np.int64)
    pos[order] = np.arange(T * k) - first              # position within its expert's run
    slot = np.where(valid & (pos < cap), flat.astype(np.int64) * cap + pos, -1)
    count = np.bincount(flat[valid], minlength=E)
    return count, slot.reshape(T, k)


@pytest.mark.parametrize("cap", [1, 3, 16, 4096])
@pytest.mark.parametrize("seed", [0, 1])
def test_positions_match_stable_sort(cap, seed):
    rng = np.random.default_rng(seed)
    T, k, E = 700, 6, 40
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)       # repeats included
    idx[rng.random(idx.shape) < 0.07] = -1
    idx[rng.random(idx.shape) < 0.03] = E + 3
    L = oracle.ll_layout(idx, E, cap)
    count, slot = _expected_by_sort(idx, E, cap)
    assert np.array_equal(L["count"], count)
    assert np.array_equal(L["slot"], slot)
    taken = slot[slot >= 0]
    assert len(np.unique(taken)) == taken.size                    # each row taken once
    tok = np.nonzero(slot >= 0)[0]
    assert np.array_equal(L["src"][taken], tok)                   # src names the token
    assert taken.size == np.minimum(count, cap).sum()             # min(count, cap) rows per expert


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_no_overflow_matches_canonical_layout(name):
    w = W.CONFIGS[name]
    idx, _ = oracle.route(W.gen_logits(w), w.G, w.TG, w.k, w.topm)
    lay = oracle.layout(idx, w.E, w.R)
    cap = w.T                                                     # a routed token names an expert once
    L = oracle.ll_layout(idx, w.E, cap)
    assert np.array_equal(L["count"], lay["cnt"])
    e = idx.astype(np.int64)
    expect = e * cap + (lay["slot"] - lay["off"][e])
    assert np.array_equal(L["slot"], expect)


def test_rejects_bad_capacity():
    with pytest.raises(ValueError):
        oracle.ll_layout(np.zeros((2, 2), np.int32), 4, 0)
