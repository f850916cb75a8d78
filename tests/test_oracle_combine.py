"""Pins for the oracle's combine: exact identities, the fp32-accumulation
error bound against an fp64 sum, torch's fp32 product, and unrouted pairs."""
import numpy as np
import torch

import oracle
import workloads as W
from checks import bf16_to_f32


def _setup(w, T):
    w = w.replace(T=T)
    idx, wt = oracle.route(W.gen_logits(w), w.G, w.TG, w.k, w.topm)
    L = oracle.layout(idx, w.E, w.R)
    y = W.gen_y(w)
    return w, wt, L["slot"], y


def test_single_expert_unit_weight_is_identity():
    y = W.gen_y(W.TINY, nrows=10)
    slot = np.arange(10, dtype=np.int32)[::-1].reshape(10, 1).copy()
    out = oracle.combine(y, slot, np.ones((10, 1), np.float32))
    assert np.array_equal(out, y[::-1])


def test_fp32_result_within_derived_bound_of_fp64_sum():
    w, wt, slot, y = _setup(W.PREFILL, T=64)
    out = bf16_to_f32(oracle.combine(y, slot, wt)).astype(np.float64)
    exact = oracle.combine_f64(y, slot, wt)
    absum = np.einsum("tj,tjc->tc", np.abs(wt.astype(np.float64)),
                      np.abs(bf16_to_f32(y[slot]).astype(np.float64)))
    # k fused multiply-adds each round once (unit 2^-24) and the final bf16
    # rounding is at most half a bf16 step (2^-8 relative to the result)
    acc_err = w.k * 2.0 ** -24 * absum
    bound = 2.0 ** -8 * (np.abs(exact) + acc_err) + acc_err + 2.0 ** -133
    assert np.all(np.abs(out - exact) <= bound)
    # and almost everywhere the bf16 result is the correctly rounded sum
    ref = oracle.bf16_from_f32(exact.astype(np.float32))
    assert (oracle.combine(y, slot, wt) == ref).mean() > 0.999


def test_matches_torch_fp32_product():
    w, wt, slot, y = _setup(W.DECODE, T=32)
    yt = torch.from_numpy(bf16_to_f32(y[slot]))          # [T, k, H]
    ref = torch.bmm(torch.from_numpy(wt).unsqueeze(1), yt).squeeze(1)
    out = bf16_to_f32(oracle.combine(y, slot, wt))
    exact = oracle.combine_f64(y, slot, wt)
    assert np.all(np.abs(out - ref.numpy()) <= 2.0 ** -7 * np.abs(exact) + 1e-5)


def test_unrouted_pairs_are_skipped():
    w, wt, slot, y = _setup(W.TINY, T=16)
    s2 = slot.copy()
    s2[:, 1] = -1
    w2 = wt.copy()
    w2[:, 1] = 0.0
    a = oracle.combine(y, s2, wt)
    b = oracle.combine(y, slot, w2)
    assert np.array_equal(a, b)
    # all pairs unrouted -> zeros
    assert np.all(oracle.combine(y, np.full_like(slot, -1), wt) == 0)
