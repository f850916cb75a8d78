"""Pins for the oracle's FP8 and BF16 dispatch: per-block closed forms,
the rounding bound of E4M3, saturation of each block's largest element,
replication to all k rows, and the dispatch -> combine round trip."""
import numpy as np
import pytest

import oracle
import workloads as W
from checks import bf16_to_f32


def _routed(w, T=None):
    w = w if T is None else w.replace(T=T)
    idx, wt = oracle.route(W.gen_logits(w), w.G, w.TG, w.k, w.topm)
    return w, idx, wt, oracle.layout(idx, w.E, w.R)


@pytest.mark.parametrize("name", ["tiny", "large"])
def test_fp8_block_closed_form(name):
    w, idx, wt, L = _routed(W.CONFIGS[name], T=64)
    x = W.gen_x(w, T=w.T)
    q, sc = oracle.dispatch_fp8(x, L["slot"], w.nrows)
    xf = bf16_to_f32(x).reshape(w.T, w.H // 128, 128)
    amax = np.abs(xf).max(-1)
    a = np.maximum(amax, np.float32(1e-4)).astype(np.float32)
    row0 = L["slot"][:, 0]
    assert np.array_equal(sc[row0], (a / np.float32(448.0)).astype(np.float32))
    inv = (np.float32(448.0) / a).astype(np.float32)
    v = (xf * inv[..., None]).astype(np.float64)
    dq = oracle.e4m3_to_f32(q[row0].ravel()).reshape(v.shape).astype(np.float64)
    # round to nearest: error at most half the E4M3 spacing at |v|
    av = np.abs(v)
    e = np.floor(np.log2(np.maximum(av, 2.0 ** -6)))
    half = 2.0 ** (e - 4)
    assert np.all(np.abs(dq - v) <= half * (1 + 1e-12))
    # each block's largest magnitude lands on +-448 (v is 448 within 2 ulp)
    big = np.abs(xf) == amax[..., None]
    assert np.all(np.abs(dq[big & (amax[..., None] >= 1e-4)]) == 448.0)


def test_fp8_rows_replicated_and_untouched_rows_kept():
    w, idx, wt, L = _routed(W.TINY)
    x = W.gen_x(w)
    slot = L["slot"].copy()
    slot[3, 1] = -1                          # drop one pair
    q0 = np.full((w.nrows, w.H), 0xAB, np.uint8)
    s0 = np.full((w.nrows, w.H // 128), -7.0, np.float32)
    q, sc = oracle.dispatch_fp8(x, slot, w.nrows, q0, s0)
    for t in range(w.T):
        rows = [r for r in slot[t] if r >= 0]
        for r in rows[1:]:
            assert np.array_equal(q[r], q[rows[0]]) and np.array_equal(sc[r], sc[rows[0]])
    dropped = L["slot"][3, 1]
    assert np.all(q[dropped] == 0xAB) and np.all(sc[dropped] == -7.0)


def test_fp8_zero_block_uses_floor():
    x = np.zeros((1, 256), np.uint16)
    x[0, 130] = 0x3F80                       # 1.0 in the second block only
    q, sc = oracle.dispatch_fp8(x, np.int32([[0]]), 1)
    assert sc[0, 0] == np.float32(np.float32(1e-4) / np.float32(448.0))
    assert np.all(q[0, :128] == 0)
    assert q[0, 130] == 0x7E and sc[0, 1] == np.float32(1.0 / 448.0)


def test_bf16_dispatch_copies_rows():
    w, idx, wt, L = _routed(W.TINY)
    x = W.gen_x(w)
    recv = oracle.dispatch_bf16(x, L["slot"], w.nrows)
    assert np.array_equal(recv[L["slot"].ravel()], np.repeat(x, w.k, axis=0))


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_dispatch_then_unweighted_combine_round_trip(name):
    # expert outputs = the dequantised payload of each receive row; with
    # w = 1/k (k a power of two) the combine returns that value exactly,
    # and with w = 1 exactly k times it
    w, idx, wt, L = _routed(W.CONFIGS[name], T=32)
    assert w.k & (w.k - 1) == 0
    x = W.gen_x(w, T=w.T)
    q, sc = oracle.dispatch_fp8(x, L["slot"], w.nrows)
    deq = oracle.e4m3_to_f32(q.ravel()).reshape(q.shape) * np.repeat(sc, 128, axis=1)
    y = oracle.bf16_from_f32(deq.astype(np.float32))
    v = y[L["slot"][:, 0]]
    out = oracle.combine(y, L["slot"], np.full((w.T, w.k), 1.0 / w.k, np.float32))
    # equal as values (a -0 payload comes back as +0: the sum starts at +0)
    assert np.array_equal(bf16_to_f32(out), bf16_to_f32(v))
    nz = bf16_to_f32(v) != 0
    assert np.array_equal(out[nz], v[nz])
    out = oracle.combine(y, L["slot"], np.ones((w.T, w.k), np.float32))
    assert np.array_equal(bf16_to_f32(out), bf16_to_f32(v) * w.k)
    # and the payload round-trips to x within the E4M3 relative step
    xf = bf16_to_f32(x)
    err = np.abs(bf16_to_f32(v) - xf)
    blk_amax = np.repeat(np.abs(xf).reshape(w.T, -1, 128).max(-1), 128, axis=1)
    assert np.all(err <= np.maximum(np.abs(xf) * (2.0 ** -4 + 2.0 ** -8), blk_amax * 2.0 ** -9 / 448 * 2 + 1e-30))
