"""Pins for the oracle's per-rank deduplicated layout and two-level combine:
hand-worked cases, a stable sort of the first picks' ranks (library routine),
the per-rank token counts of the canonical layout, the one-rank case
(equal to the flat combine bit for bit), the one-expert-per-rank case
(numpy fp32 products and sums), and the fp64 bound."""
import numpy as np
import pytest

import oracle
import workloads as W
from checks import bf16_to_f32, golden_lines


def _ints(s):
    return [int(v) for v in s.split()]


def _golden():
    for line in golden_lines("rank_layout_cases.txt"):
        head, idx, cnt, off, rslot, rtok = [p.strip() for p in line.split("|")]
        E, R = _ints(head)
        yield (E, R, np.array([_ints(r) for r in idx.split(";")], np.int32), _ints(cnt), _ints(off),
               np.array([_ints(r) for r in rslot.split(";")], np.int32), _ints(rtok))


@pytest.mark.parametrize("case", list(_golden()))
def test_hand_worked_cases(case):
    E, R, idx, cnt, off, rslot, rtok = case
    L = oracle.rank_layout(idx, E, R)
    assert L["rank_count"].tolist() == cnt
    assert L["rank_offset"].tolist() == off
    assert np.array_equal(L["rank_slot"], rslot)
    assert L["rank_token"].tolist() == rtok


def _first_pick_ranks(idx, E, R):
    """rank of each pick if it is the token's first pick on that rank, else R
    (numpy: first occurrence per token via np.unique)."""
    T, k = idx.shape
    EPR = E // R
    key = np.full((T, k), R, np.int64)
    for t in range(T):
        valid = (idx[t] >= 0) & (idx[t] < E)
        ranks = np.where(valid, idx[t] // EPR, -1)
        u, first = np.unique(ranks, return_index=True)
        for r, j in zip(u, first):
            if r >= 0:
                key[t, j] = r
    return key


@pytest.mark.parametrize("E,R", [(64, 8), (64, 64), (48, 1), (256, 32)])
def test_rank_rows_match_stable_sort(E, R):
    rng = np.random.default_rng(E + R)
    T, k = 500, 8
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    L = oracle.rank_layout(idx, E, R)
    key = _first_pick_ranks(idx, E, R).ravel()
    used = int((key < R).sum())
    order = np.argsort(key, kind="stable")[:used]
    slot = np.full(T * k, -1, np.int64)
    slot[order] = np.arange(used)
    assert np.array_equal(L["rank_slot"].ravel(), slot)
    cnt = np.bincount(key[key < R], minlength=R)
    assert np.array_equal(L["rank_count"], cnt)
    assert np.array_equal(L["rank_offset"], np.concatenate([[0], np.cumsum(cnt)]))
    assert np.array_equal(L["rank_token"][:used], order // k)
    # rows per rank = distinct tokens per rank = the canonical layout's ntok_rank
    assert np.array_equal(L["rank_count"], oracle.layout(idx, E, R)["ntok_rank"])


def _routed(w, T=None):
    w = w if T is None else w.replace(T=T)
    lg = W.gen_logits(w)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    lay = oracle.layout(idx, w.E, w.R)
    return w, idx, wt, lay, W.gen_y(w)


def test_one_rank_equals_flat_combine():
    # R = 1: a token's picks all sit on one rank, so its partial row is the
    # flat combine's fp32 chain rounded once, and summing one partial changes
    # nothing: the two-level result is the flat combine bit for bit
    w, idx, wt, lay, y = _routed(W.TINY.replace(R=1))
    rl = oracle.rank_layout(idx, w.E, 1)
    part = oracle.combine_rank_partial(y, idx, lay["slot"], wt, rl["rank_slot"], w.E, 1, w.nrows)
    flat = oracle.combine(y, lay["slot"], wt)
    two = oracle.combine_ranks(part, rl["rank_slot"])
    assert np.array_equal(two, flat)
    assert np.array_equal(part[rl["rank_slot"][:, 0]], flat)


def test_one_expert_per_rank_reduces_to_products_and_sums():
    # R = E with distinct picks: partial row of pick j = bf16(fp32(w_j * y_j));
    # the final row sums those in pick order in fp32 and rounds once
    w, idx, wt, lay, y = _routed(W.TINY.replace(R=W.TINY.E))
    rl = oracle.rank_layout(idx, w.E, w.E)
    assert np.all(rl["rank_slot"] >= 0)
    part = oracle.combine_rank_partial(y, idx, lay["slot"], wt, rl["rank_slot"], w.E, w.E, w.nrows)
    yf = bf16_to_f32(y)
    for j in range(w.k):
        prod = (wt[:, j:j + 1].astype(np.float32) * yf[lay["slot"][:, j]]).astype(np.float32)
        assert np.array_equal(part[rl["rank_slot"][:, j]], oracle.bf16_from_f32(prod))
    acc = np.zeros((w.T, w.H), np.float32)
    for j in range(w.k):
        acc = (acc + bf16_to_f32(part[rl["rank_slot"][:, j]])).astype(np.float32)
    assert np.array_equal(oracle.combine_ranks(part, rl["rank_slot"]), oracle.bf16_from_f32(acc))


def test_two_level_combine_within_bound_of_exact_sum():
    w, idx, wt, lay, y = _routed(W.PREFILL, T=128)
    rl = oracle.rank_layout(idx, w.E, w.R)
    part = oracle.combine_rank_partial(y, idx, lay["slot"], wt, rl["rank_slot"], w.E, w.R, w.nrows)
    two = bf16_to_f32(oracle.combine_ranks(part, rl["rank_slot"])).astype(np.float64)
    exact = oracle.combine_f64(y, lay["slot"], wt)
    yabs = np.abs(bf16_to_f32(y)).astype(np.float64)
    mag = np.zeros_like(exact)
    for j in range(w.k):
        mag += np.abs(wt[:, j:j + 1]).astype(np.float64) * yabs[lay["slot"][:, j]]
    # each partial: k fp32 fmas (k 2^-24) then one bf16 rounding (2^-8);
    # the sum of <= k partials in fp32 (k 2^-24), then one bf16 rounding
    u8, u24 = 2.0 ** -8, 2.0 ** -24
    bound = (u8 + 2 * w.k * u24) * (1 + u8) * mag + u8 * np.abs(exact) + 1e-30
    assert np.all(np.abs(two - exact) <= bound)


def test_deduplicated_dispatch_rows():
    # dispatch through rank_slot writes each token once per rank it needs:
    # the rows equal the flat dispatch's rows of the same token
    w, idx, wt, lay, _ = _routed(W.PREFILL, T=64)
    x = W.gen_x(w)
    rl = oracle.rank_layout(idx, w.E, w.R)
    used = int(rl["rank_offset"][-1])
    qd, sd = oracle.dispatch_fp8(x, rl["rank_slot"], w.nrows)
    qf, sf = oracle.dispatch_fp8(x, lay["slot"], w.nrows)
    tok = rl["rank_token"][:used]
    first_flat_row = lay["slot"][np.arange(w.T), 0]
    assert np.array_equal(qd[:used], qf[first_flat_row[tok]])
    assert np.array_equal(sd[:used], sf[first_flat_row[tok]])
    assert used < w.T * w.k
