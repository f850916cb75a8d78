"""Pins for the oracle's routing layout: a stable sort of the flattened
expert ids (library routine), bincount/cumsum, brute-force rank sets, and
conservation invariants."""
import numpy as np
import pytest

import oracle
import workloads as W


def _check_against_stable_sort(idx, E, R):
    T, k = idx.shape
    L = oracle.layout(idx, E, R)
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    # counts and offsets
    cnt = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(L["cnt"], cnt)
    assert np.array_equal(L["off"], np.concatenate([[0], np.cumsum(cnt)]))
    # receive rows = pairs stably sorted by expert; slot is the inverse map
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")[: valid.sum()]
    assert np.array_equal(L["recv_token"][: valid.sum()], order // k)
    assert np.all(L["recv_token"][valid.sum():] == -1)
    slot = np.full(T * k, -1, np.int64)
    slot[order] = np.arange(valid.sum())
    assert np.array_equal(L["slot"].ravel(), slot)
    # distinct tokens per virtual rank, by explicit sets
    EPR = E // R
    ntok = [len({t for t in range(T) for j in range(k) if valid[t * k + j] and flat[t * k + j] // EPR == r})
            for r in range(R)]
    assert L["ntok_rank"].tolist() == ntok
    return L


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed_literal"])
def test_layout_from_routed_workloads(name):
    w = W.CONFIGS[name]
    if w.T > 1024:
        w = w.replace(T=1024)
    idx, _ = oracle.route(W.gen_logits(w), w.G, w.TG, w.k, w.topm)
    _check_against_stable_sort(idx, w.E, w.R)


def test_layout_with_unrouted_and_out_of_range_entries():
    rng = np.random.default_rng(5)
    T, k, E, R = 200, 6, 48, 8
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    drop = rng.random((T, k)) < 0.15
    idx[drop] = -1
    idx[rng.random((T, k)) < 0.05] = E + 3
    L = _check_against_stable_sort(idx, E, R)
    assert np.all(L["slot"][idx < 0] == -1) and np.all(L["slot"][idx >= E] == -1)


def test_conservation_invariants_prefill():
    w = W.PREFILL
    idx, _ = oracle.route(W.gen_logits(w), w.G, w.TG, w.k, w.topm)
    L = oracle.layout(idx, w.E, w.R)
    assert L["cnt"].sum() == w.T * w.k
    assert L["off"][-1] == w.T * w.k
    s = L["slot"].ravel()
    assert np.array_equal(np.sort(s), np.arange(w.T * w.k))          # bijection
    e = idx.ravel()
    assert np.all((s >= L["off"][e]) & (s < L["off"][e + 1]))         # own segment
    assert np.all(np.bincount(L["recv_token"], minlength=w.T) == w.k)  # k rows per token
    assert np.all(L["ntok_rank"] <= w.T)
    # ranks receive between 1 and k/1 copies per token they serve
    EPR = w.E // w.R
    rows_rank = np.add.reduceat(L["cnt"], np.arange(0, w.E, EPR))
    assert np.all(rows_rank >= L["ntok_rank"])
    # within an expert's segment tokens ascend
    rt = L["recv_token"]
    for ex in range(w.E):
        seg = rt[L["off"][ex]:L["off"][ex + 1]]
        assert np.all(np.diff(seg) > 0)


def test_layout_empty_and_degenerate():
    L = oracle.layout(np.zeros((0, 4), np.int32), 16, 4)
    assert L["cnt"].sum() == 0 and L["off"].tolist() == [0] * 17 and L["ntok_rank"].sum() == 0
    # every token to the same k experts (the literal-skew shape)
    idx = np.tile(np.arange(4, dtype=np.int32), (100, 1))
    L = _check_against_stable_sort(idx, 16, 4)
    assert L["cnt"][:4].tolist() == [100] * 4


def test_layout_rejects_bad_rank_split():
    with pytest.raises(ValueError):
        oracle.layout(np.zeros((2, 2), np.int32), 16, 3)
