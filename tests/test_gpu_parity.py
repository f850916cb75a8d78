"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Bar: bit-exact routing indices and weights, layout counts, offsets, slots
and receive-row owners, FP8 codes and scales, BF16 dispatch; combine output
within 1 bf16 ulp (counted on monotone-mapped bf16 patterns, +-0 equal) of
the oracle's fp32 result; every run is expected to be bit-exact there too and
the count of differing elements is reported."""
import numpy as np
import pytest
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W
from checks import bf16_to_f32, bf16_ulp_diff
from pipeline import gpu_pipeline, inputs, oracle_pipeline, to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def assert_same(name, got, ref):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    assert bad.size == 0, "%s: %d of %d differ, first at %s: got %s want %s" % (
        name, bad.size, got.size, np.unravel_index(bad[0], got.shape), got.ravel()[bad[0]], ref.ravel()[bad[0]])


def assert_combine(got, ref, tol_ulp=1):
    d = bf16_ulp_diff(got, ref)
    nan_g, nan_r = np.isnan(bf16_to_f32(got)), np.isnan(bf16_to_f32(ref))
    assert np.array_equal(nan_g, nan_r)
    d = np.where(nan_g, 0, d)
    say("combine: %d of %d elements differ from the oracle, max %d ulp" % ((d > 0).sum(), d.size, d.max()))
    assert d.max() <= tol_ulp


def assert_parity(g, o, fp8=True, rows=None):
    for key in ("idx", "w", "cnt", "off", "ntok_rank", "slot", "recv_token"):
        assert_same(key, g[key], o[key])
    sel = slice(None) if rows is None else rows
    assert_same("recv", g["recv"][sel], o["recv"][sel])
    if fp8:
        assert_same("scales", g["sc"][sel], o["sc"][sel])
    assert_combine(g["out"], o["out"])


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "skewed_literal"])
def test_pipeline_parity(name):
    w = W.CONFIGS[name]
    say("parity", name, w)
    lg, x, y = inputs(w)
    g = gpu_pipeline(w, lg, x, y)
    o = oracle_pipeline(w, lg, x, y)
    assert_parity(g, o)
    if name == "skewed":
        load = o["cnt"] / o["cnt"].mean()
        say("skewed: expert load max/mean %.2f" % load.max())


def test_bf16_dispatch_parity():
    w = W.PREFILL.replace(T=1024)
    say("bf16 dispatch", w)
    lg, x, y = inputs(w)
    g = gpu_pipeline(w, lg, x, y, recv_dtype="bf16")
    o = oracle_pipeline(w, lg, x, y, recv_dtype="bf16")
    assert_parity(g, o, fp8=False)


@pytest.mark.parametrize("recv_dtype", ["fp8", "bf16"])
def test_large_batch_full(recv_dtype):
    # full size on the GPU (the only workload on the XCD-ordered dispatch
    # path, and where BF16 dispatch is timed); every integer output, every
    # receive row and scale and every output element against the oracle,
    # which runs on chunks of 2048 tokens to bound host memory (dispatch and
    # combine are per token, so a chunk's oracle rows are its tokens' rows)
    w = W.LARGE
    say("large", recv_dtype, w)
    lg, x, y = inputs(w)
    g = gpu_pipeline(w, lg, x, y, recv_dtype=recv_dtype)
    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    assert_same("idx", g["idx"], idx)
    assert_same("w", g["w"], wt)
    lay = oracle.layout(idx, w.E, w.R)
    for key in ("cnt", "off", "ntok_rank", "slot", "recv_token"):
        assert_same(key, g[key], lay[key])
    slot = lay["slot"]
    # the chunks below cover every receive row exactly once
    assert np.array_equal(np.sort(slot.ravel()), np.arange(w.nrows, dtype=np.int32))
    chunk = 2048
    diff, worst = 0, 0
    for t0 in range(0, w.T, chunk):
        t1 = min(w.T, t0 + chunk)
        sub = w.replace(T=t1 - t0)
        local = np.arange(sub.nrows, dtype=np.int32).reshape(sub.T, sub.k)
        rows = slot[t0:t1].ravel()
        if recv_dtype == "fp8":
            q, sc = oracle.dispatch_fp8(x[t0:t1], local, sub.nrows)
            assert_same("recv tokens %d..%d" % (t0, t1), g["recv"][rows], q)
            assert_same("scales tokens %d..%d" % (t0, t1), g["sc"][rows], sc)
        else:
            r = oracle.dispatch_bf16(x[t0:t1], local, sub.nrows)
            assert_same("recv tokens %d..%d" % (t0, t1), g["recv"][rows], r)
        out = oracle.combine(y[rows], local, wt[t0:t1])
        d = bf16_ulp_diff(g["out"][t0:t1], out)
        diff += int((d > 0).sum())
        worst = max(worst, int(d.max()))
    say("large combine: %d of %d elements differ from the oracle, max %d ulp" % (diff, w.T * w.H, worst))
    assert worst <= 1


EDGE = {
    "one_token": W.PREFILL.replace(T=1),
    "ragged_77": W.PREFILL.replace(T=77),
    "ragged_2049": W.PREFILL.replace(T=2049, H=1024),
    "h128": W.TINY.replace(H=128, T=300),
    "h16384": W.PREFILL.replace(H=16384, T=40),
    "e96_g4": W.Workload("e96", T=333, H=384, E=96, G=4, TG=2, k=6, R=12, m=3, seed=7),
    "e1024_k32": W.Workload("e1024", T=150, H=256, E=1024, G=64, TG=8, k=32, R=64, m=4, seed=8),
    "k1_g1": W.Workload("k1", T=200, H=256, E=16, G=1, TG=1, k=1, R=16, seed=9),
    "tg1_m8": W.Workload("tg1", T=100, H=512, E=64, G=4, TG=1, k=16, R=2, m=8, seed=10),
    "e8_odd": W.Workload("e8", T=64, H=128, E=8, G=2, TG=2, k=3, R=1, seed=11),
    # gate kernel branches: a 64-expert group (merge across the two half-waves),
    # one-expert groups (no merge step), m = 1 with a group limit, E < 64
    "gs64": W.Workload("gs64", T=300, H=256, E=256, G=4, TG=2, k=8, R=8, m=2, seed=13),
    "gs1": W.Workload("gs1", T=300, H=256, E=16, G=16, TG=5, k=4, R=4, seed=14),
    "m1_tg3": W.Workload("m1", T=300, H=256, E=64, G=8, TG=3, k=6, R=8, m=1, seed=15),
    "e32_gs8": W.Workload("e32", T=129, H=128, E=32, G=4, TG=3, k=5, R=2, seed=16),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_shapes(name):
    w = EDGE[name]
    say("edge", name, w)
    lg, x, y = inputs(w)
    g = gpu_pipeline(w, lg, x, y)
    o = oracle_pipeline(w, lg, x, y)
    assert_parity(g, o)


def test_zero_tokens():
    w = W.PREFILL.replace(T=0)
    say("zero tokens", w)
    cfg = ep.Config.of(w)
    idx, wt = ep.route(cfg, torch.empty((0, w.E), dtype=torch.float32, device="cuda"))
    lay = ep.get_layout(cfg, idx)
    ep.dispatch(cfg, torch.empty((0, w.H), dtype=torch.bfloat16, device="cuda"), lay["slot"])
    out = ep.combine(cfg, torch.empty((0, w.H), dtype=torch.bfloat16, device="cuda"), lay["slot"], wt)
    torch.cuda.synchronize()
    assert out.shape == (0, w.H)
    assert to_host(lay["cnt"]).sum() == 0 and to_host(lay["off"]).tolist() == [0] * (w.E + 1)
    assert to_host(lay["ntok_rank"]).sum() == 0


def test_unrouted_and_repeated_entries():
    # layout, dispatch and combine fed a hand-made topk_idx with -1, >= E
    # and repeated experts
    w = W.Workload("holes", T=500, H=512, E=48, G=4, TG=4, k=6, R=8, seed=12)
    say("holes", w)
    rng = np.random.default_rng(12)
    idx = rng.integers(0, w.E, size=(w.T, w.k)).astype(np.int32)   # repeats happen
    idx[rng.random(idx.shape) < 0.1] = -1
    idx[rng.random(idx.shape) < 0.03] = w.E + 5
    wt = rng.random((w.T, w.k)).astype(np.float32)
    x, y = W.gen_x(w), W.gen_y(w)
    cfg = ep.Config.of(w)
    lay = ep.get_layout(cfg, to_dev(idx))
    ol = oracle.layout(idx, w.E, w.R)
    for key in ("cnt", "off", "ntok_rank", "slot", "recv_token"):
        assert_same(key, to_host(lay[key]), ol[key])
    fill = torch.full((w.nrows, w.H), 0x5A, dtype=torch.uint8, device="cuda")
    fsc = torch.full((w.nrows, w.H // 128), -3.0, dtype=torch.float32, device="cuda")
    recv, sc = ep.dispatch(cfg, to_dev(x, torch.bfloat16), lay["slot"], "fp8", fill, fsc)
    q0 = np.full((w.nrows, w.H), 0x5A, np.uint8)
    s0 = np.full((w.nrows, w.H // 128), -3.0, np.float32)
    q, s = oracle.dispatch_fp8(x, ol["slot"], w.nrows, q0, s0)
    assert_same("recv", to_host(recv), q)
    assert_same("scales", to_host(sc), s)
    out = ep.combine(cfg, to_dev(y, torch.bfloat16), lay["slot"], to_dev(wt))
    assert_combine(to_host(out), oracle.combine(y, ol["slot"], wt))


@pytest.mark.parametrize("T,E,k,R", [
    (127, 256, 8, 32), (128, 256, 8, 32), (129, 256, 8, 32),   # one workgroup up to 1024 pairs, launches above
    (128, 1024, 8, 64), (32, 1024, 32, 64), (33, 1024, 32, 64),  # four-wave workgroups (E = 1024), k = 32
    (1, 256, 8, 32), (170, 48, 6, 8),
])
def test_layout_around_one_workgroup_limit(T, E, k, R):
    # layout and rank layout of a hand-made topk_idx (unrouted -1 and >= E
    # entries, repeated experts) on both sides of the one-workgroup size
    w = W.Workload("lim", T=T, H=128, E=E, G=4, TG=4, k=k, R=R, seed=T * 7 + k)
    say("layout limit", w)
    rng = np.random.default_rng(w.seed)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.08] = -1
    idx[rng.random(idx.shape) < 0.02] = E + 3
    cfg = ep.Config.of(w)
    lay = ep.get_layout(cfg, to_dev(idx))
    rl = ep.get_rank_layout(cfg, to_dev(idx))
    ol = oracle.layout(idx, E, R)
    orl = oracle.rank_layout(idx, E, R)
    for key in ("cnt", "off", "ntok_rank", "slot", "recv_token"):
        assert_same(key, to_host(lay[key]), ol[key])
    for key in ("rank_count", "rank_offset", "rank_slot", "rank_token"):
        assert_same(key, to_host(rl[key]), orl[key])


def test_fp8_cast_covers_every_bf16_value():
    # blocks whose largest magnitude is A and whose other 127 values sweep
    # every bf16 pattern with |v| <= A; inv = 448 / max(A, 1e-4) takes
    # several mantissas, so x * inv covers many fp32 patterns
    H = 7168
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f32(b)
    blocks = []
    for A in (448.0, 1.0, 3.140625, 0.69921875, 100.0, 2.0 ** -20, 1e-3, 5e-5):
        a16 = oracle.bf16_from_f32(np.float32([A]))[0]
        A = bf16_to_f32(np.uint16([a16]))[0]
        pool = b[np.isfinite(vals) & (np.abs(vals) <= A)]
        pad = (-len(pool)) % 127
        pool = np.concatenate([pool, pool[:pad]])
        body = pool.reshape(-1, 127)
        blocks.append(np.concatenate([np.full((len(body), 1), a16, np.uint16), body], axis=1))
    blocks = np.concatenate(blocks)
    pad = (-len(blocks)) % (H // 128)
    blocks = np.concatenate([blocks, blocks[:pad]])
    x = blocks.reshape(-1, H)
    T = x.shape[0]
    w = W.Workload("fp8sweep", T=T, H=H, E=8, G=1, TG=1, k=1, R=1, seed=0)
    say("fp8 sweep", T, "tokens")
    slot = np.arange(T, dtype=np.int32).reshape(T, 1)
    cfg = ep.Config.of(w)
    recv, sc = ep.dispatch(cfg, to_dev(x, torch.bfloat16), to_dev(slot))
    q, s = oracle.dispatch_fp8(x, slot, T)
    assert_same("recv", to_host(recv), q)
    assert_same("scales", to_host(sc), s)


def test_bf16_rounding_and_ties():
    # k = 2, unit weights: out = bf16(y0 + y1); pairs built so that the fp32
    # sum lands exactly halfway between bf16 neighbours, and random pairs
    H = 256
    rng = np.random.default_rng(3)
    base = rng.integers(0x3C00, 0x4400, size=4096).astype(np.uint16)      # 2^-7 .. 2^1
    e = ((base.astype(np.int32) >> 7) & 0xFF) - 8                         # half-ulp exponent
    half = (e.astype(np.uint32) << 7).astype(np.uint16)                   # 2^(E-8), exact
    odd = rng.integers(0, 2 ** 16, size=4096).astype(np.uint16)
    y0 = np.concatenate([base, odd])
    y1 = np.concatenate([half, rng.integers(0, 2 ** 16, size=4096).astype(np.uint16)])
    keep = np.isfinite(bf16_to_f32(y0)) & np.isfinite(bf16_to_f32(y1))
    y0, y1 = y0[keep], y1[keep]
    n = (len(y0) // H) * H
    T = n // H
    y = np.stack([y0[:n].reshape(T, H), y1[:n].reshape(T, H)], axis=1).reshape(2 * T, H)
    slot = np.arange(2 * T, dtype=np.int32).reshape(T, 2)
    wt = np.ones((T, 2), np.float32)
    w = W.Workload("ties", T=T, H=H, E=8, G=1, TG=1, k=2, R=1, seed=0)
    say("bf16 ties", T, "tokens")
    out = ep.combine(ep.Config.of(w), to_dev(y, torch.bfloat16), to_dev(slot), to_dev(wt))
    ref = oracle.combine(y, slot, wt)
    assert_same("out", to_host(out), ref)


def test_sigmoid_over_wide_logit_range():
    # logits spread over [-100, 100] (both saturation regions and every
    # binade in between); selection and weights must match bit for bit
    w = W.Workload("wide", T=4096, H=128, E=64, G=4, TG=2, k=4, R=4, seed=0)
    rng = np.random.default_rng(4)
    lg = (rng.standard_normal((w.T, w.E)) * np.exp(rng.uniform(-12, 4.6, (w.T, w.E)))).astype(np.float32)
    lg = np.clip(lg, -100, 100).astype(np.float32)
    say("wide logits", w)
    idx, wt = ep.route(ep.Config.of(w), to_dev(lg))
    oi, ow = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    assert_same("idx", to_host(idx), oi)
    assert_same("w", to_host(wt), ow)


def test_deterministic_and_in_bounds():
    # two runs bit-identical; guard rows after every output untouched
    w = W.PREFILL.replace(T=2048)
    say("determinism", w)
    lg, x, y = inputs(w)
    cfg = ep.Config.of(w)
    G = 8
    runs = []
    for _ in range(2):
        idx_b = torch.full((w.T + G, w.k), 0x7A7A7A7A, dtype=torch.int32, device="cuda")
        w_b = torch.full((w.T + G, w.k), 1.5, dtype=torch.float32, device="cuda")
        idx, wt = ep.route(cfg, to_dev(lg), idx_b[:w.T], w_b[:w.T])
        outs = {k: torch.full((n + G,), -77, dtype=torch.int32, device="cuda")
                for k, n in (("cnt", w.E), ("ntok_rank", w.R), ("off", w.E + 1), ("recv_token", w.nrows))}
        slot_b = torch.full((w.T + G, w.k), -77, dtype=torch.int32, device="cuda")
        lay = ep.get_layout(cfg, idx, {**{k: v[:-G] for k, v in outs.items()}, "slot": slot_b[:w.T]})
        recv_b = torch.full((w.nrows + G, w.H), 0x33, dtype=torch.uint8, device="cuda")
        sc_b = torch.full((w.nrows + G, w.H // 128), 9.0, dtype=torch.float32, device="cuda")
        ep.dispatch(cfg, to_dev(x, torch.bfloat16), lay["slot"], "fp8", recv_b[:w.nrows], sc_b[:w.nrows])
        out_b = torch.full((w.T + G, w.H), 1.0, dtype=torch.bfloat16, device="cuda")
        ep.combine(cfg, to_dev(y, torch.bfloat16), lay["slot"], wt, out_b[:w.T])
        torch.cuda.synchronize()
        assert torch.all(idx_b[w.T:] == 0x7A7A7A7A) and torch.all(w_b[w.T:] == 1.5)
        assert torch.all(slot_b[w.T:] == -77)
        for v in outs.values():
            assert torch.all(v[-G:] == -77)
        assert torch.all(recv_b[w.nrows:] == 0x33) and torch.all(sc_b[w.nrows:] == 9.0)
        assert torch.all(out_b[w.T:] == 1.0)
        runs.append([to_host(t) for t in (idx_b, w_b, slot_b, recv_b, sc_b, out_b, *outs.values())])
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
