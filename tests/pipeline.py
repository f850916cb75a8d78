"""Runs the HIP path (through the C ABI binding) and the oracle on the same
seeded inputs, for the parity tests, the smoke check and the benchmark."""
from __future__ import annotations

import numpy as np
import torch

import combine_group_limited_amd as ep
import oracle
import workloads as W


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
        return t.numpy().view(np.uint16)
    return t.numpy()


def gpu_pipeline(w: W.Workload, logits: np.ndarray, x: np.ndarray, y: np.ndarray, recv_dtype="fp8"):
    """All four steps on the GPU; returns numpy copies of every output."""
    cfg = ep.Config.of(w)
    lg = to_dev(logits)
    xd = to_dev(x, torch.bfloat16)
    yd = to_dev(y, torch.bfloat16)
    idx, wt = ep.route(cfg, lg)
    lay = ep.get_layout(cfg, idx)
    recv, sc = ep.dispatch(cfg, xd, lay["slot"], recv_dtype)
    out = ep.combine(cfg, yd, lay["slot"], wt)
    torch.cuda.synchronize()
    res = dict(idx=to_host(idx), w=to_host(wt), out=to_host(out), recv=to_host(recv))
    res.update({k: to_host(v) for k, v in lay.items()})
    if sc is not None:
        res["sc"] = to_host(sc)
    return res


def oracle_pipeline(w: W.Workload, logits: np.ndarray, x: np.ndarray, y: np.ndarray, recv_dtype="fp8"):
    idx, wt = oracle.route(logits, w.G, w.TG, w.k, w.topm)
    lay = oracle.layout(idx, w.E, w.R)
    res = dict(idx=idx, w=wt)
    res.update(lay)
    if recv_dtype == "fp8":
        res["recv"], res["sc"] = oracle.dispatch_fp8(x, lay["slot"], w.nrows)
    else:
        res["recv"] = oracle.dispatch_bf16(x, lay["slot"], w.nrows)
    res["out"] = oracle.combine(y, lay["slot"], wt)
    return res


def inputs(w: W.Workload):
    return W.gen_logits(w), W.gen_x(w), W.gen_y(w)
