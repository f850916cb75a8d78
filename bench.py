#!/usr/bin/env python3
"""Benchmark of the MoE routing -> FP8 dispatch -> BF16 combine path on one
MI355X.

One step = ep_route + ep_get_layout + ep_dispatch (FP8 E4M3, 1x128 scales)
+ ep_combine over one batch of seeded synthetic input already resident in
HBM (4096 tokens x 7168 hidden, 256 experts in 8 groups, top-4 groups,
top-8 experts, 32 virtual ranks by default).  Expert outputs for the combine
are a resident synthetic buffer (the expert computation is not part of the
path).

Every buffer exists in several copies used round-robin, so that each step
reads its inputs from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line.  `value` is dispatch+combine algorithmic bytes divided
by the summed average durations of the dispatch and combine kernels, from
HIP events recorded on the launch stream over the timed steps.  The
`roofline` object reports the dominant kernel (combine); `cpu_baseline`
times the single-threaded CPU oracle on the same batch.

usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5]
                       [--config prefill] [--sets N] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published

# hipEventCreateWithFlags flag: the event's record does not release to system
# scope, so it adds no L2 write-back to the interval it closes (the GPU-side
# timestamps are the same).  Back-to-back launches of the combine kernel and
# per-launch events with this flag agree within ~0.3%; default events read
# ~2 us longer per launch.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """HIP events created and recorded through the HIP runtime that torch
    loaded (the one libep.so binds to), on the caller's stream handle."""

    def __init__(self):
        import ctypes
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        H = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
        vp = ctypes.c_void_p
        H.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        H.hipEventRecord.argtypes = [vp, vp]
        H.hipEventSynchronize.argtypes = [vp]
        H.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        H.hipEventDestroy.argtypes = [vp]
        self.H, self.ct = H, ctypes

    def create(self, n):
        evs = []
        for _ in range(n):
            e = self.ct.c_void_p()
            rc = self.H.hipEventCreateWithFlags(self.ct.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
            evs.append(e)
        return evs

    def record(self, e, stream_handle):
        rc = self.H.hipEventRecord(e, self.ct.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def seconds(self, a, b):
        self.H.hipEventSynchronize(b)
        f = self.ct.c_float()
        rc = self.H.hipEventElapsedTime(self.ct.byref(f), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return f.value * 1e-3

    def destroy(self, evs):
        for e in evs:
            self.H.hipEventDestroy(e)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="prefill")
    ap.add_argument("--sets", type=int, default=0,
                    help="copies of all buffers used round-robin (0: enough for >= 2 GiB between reuses)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM counters)")
    return ap.parse_args()


def copy_probe():
    """A plain copy of known size: 5 x 1 GiB device-to-device copies.  Its
    FETCH_SIZE / WRITE_SIZE readings give the factor between those counters
    and bytes actually moved."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.copy_(a)
    torch.cuda.synchronize()
    s.record()
    for _ in range(5):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 5 * 1e-3
    print(json.dumps({"kind": "copy_probe", "bytes_read": n, "bytes_written": n,
                      "us": round(t * 1e6, 1), "gbs_read_plus_write": round(2 * n / t / 1e9, 1)}), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe()

    import numpy as np
    import torch

    import combine_group_limited_amd as ep
    from combine_group_limited_amd import _lib as L
    import workloads as W

    w = W.CONFIGS[args.config]
    cfg = ep.Config.of(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    # Resident inputs and outputs, in `nsets` copies used round-robin so that
    # no step finds its data in the 256 MB Infinity Cache or the L2s: between
    # two uses of a copy the other steps move >= 2 GiB through memory.
    lg_np, x_np, y_np = W.gen_logits(w), W.gen_x(w), W.gen_y(w)
    set_bytes = w.bytes_dispatch_fp8() + w.bytes_combine() + w.bytes_route()
    nsets = args.sets or int(min(256, max(4, -(-(2 << 30) // set_bytes))))
    logits0 = torch.from_numpy(lg_np).to(dev)
    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    y0 = torch.from_numpy(y_np.view(np.int16)).view(torch.bfloat16).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    ws = torch.empty(max(16, ep.layout_workspace_bytes(cfg)), dtype=torch.uint8, device=dev)
    sets = []
    for i in range(nsets):
        b = dict(
            logits=logits0 if i == 0 else logits0.clone(),
            x=x0 if i == 0 else x0.clone(),
            y=y0 if i == 0 else y0.clone(),
            idx=torch.empty((w.T, w.k), **i32),
            wt=torch.empty((w.T, w.k), dtype=torch.float32, device=dev),
            cnt=torch.empty(w.E, **i32), ntok=torch.empty(w.R, **i32), off=torch.empty(w.E + 1, **i32),
            slot=torch.empty((w.T, w.k), **i32), recv_token=torch.empty(w.nrows, **i32),
            recv=torch.empty((w.nrows, w.H), dtype=torch.uint8, device=dev),
            scales=torch.empty((w.nrows, w.H // 128), dtype=torch.float32, device=dev),
            out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev))
        sets.append(b)

    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    lib = L.lib()
    c = cfg.c()
    cp = ctypes.byref(c)
    # validate once through the checked binding, then call the C ABI directly
    for b in sets:
        ep.route(cfg, b["logits"], b["idx"], b["wt"])
        ep.get_layout(cfg, b["idx"], dict(cnt=b["cnt"], ntok_rank=b["ntok"], off=b["off"], slot=b["slot"],
                                          recv_token=b["recv_token"]), ws)
        ep.dispatch(cfg, b["x"], b["slot"], "fp8", b["recv"], b["scales"])
        ep.combine(cfg, b["y"], b["slot"], b["wt"], b["out"])
    torch.cuda.synchronize()
    ptr = [{k: v.data_ptr() for k, v in b.items()} for b in sets]

    def check(rc, name):
        if rc != 0:
            raise RuntimeError("%s failed: %s" % (name, lib.ep_strerror(rc).decode()))

    stages = ("route", "layout", "dispatch", "combine")
    nws = ws.numel()
    hev = HipEvents()

    def step(i, ev):
        p = ptr[i % nsets]
        hev.record(ev[0], sh)
        check(lib.ep_route(cp, p["logits"], p["idx"], p["wt"], sh), "ep_route")
        hev.record(ev[1], sh)
        check(lib.ep_get_layout(cp, p["idx"], p["cnt"], p["ntok"], p["off"], p["slot"], p["recv_token"],
                                ws.data_ptr(), nws, sh), "ep_get_layout")
        hev.record(ev[2], sh)
        check(lib.ep_dispatch(cp, p["x"], p["slot"], L.EP_RECV_FP8_E4M3, p["recv"], p["scales"], sh),
              "ep_dispatch")
        hev.record(ev[3], sh)
        check(lib.ep_combine(cp, p["y"], p["slot"], p["wt"], p["out"], sh), "ep_combine")
        hev.record(ev[4], sh)

    warm = [hev.create(5) for _ in range(max(args.warmup, 0))]
    for i, ev in enumerate(warm):
        step(i, ev)
    torch.cuda.synchronize()

    evs = [hev.create(5) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, ev in enumerate(evs):
        step(args.warmup + i, ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dur = {s: [] for s in stages}
    for ev in evs:
        for i, s in enumerate(stages):
            dur[s].append(hev.seconds(ev[i], ev[i + 1]))
    for ev in warm + evs:
        hev.destroy(ev)
    avg = {s: float(np.mean(v)) for s, v in dur.items()}
    med = {s: float(np.median(v)) for s, v in dur.items()}

    bytes_ = dict(route=w.bytes_route(), layout=w.bytes_layout(), dispatch=w.bytes_dispatch_fp8(),
                  combine=w.bytes_combine())
    dc_bytes = bytes_["dispatch"] + bytes_["combine"]
    dc_time = avg["dispatch"] + avg["combine"]
    value = dc_bytes / dc_time / 1e9
    per_kernel = {s: dict(avg_us=avg[s] * 1e6, median_us=med[s] * 1e6,
                          algorithmic_bytes=bytes_[s], gbs=bytes_[s] / avg[s] / 1e9,
                          frac=bytes_[s] / avg[s] / 1e9 / HBM_PEAK_GBS) for s in stages}

    traffic = _recorded_traffic(args.config)

    comb_gbs = bytes_["combine"] / avg["combine"] / 1e9
    rec = {
        "metric": "dispatch+combine HBM GB/s and % of peak at 4096 tok x 7168 hidden top-8",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E, "groups": w.G,
                   "topk_groups": w.TG, "topk": w.k, "virtual_ranks": w.R,
                   "dispatch": "fp8_e4m3_1x128_fp32_scales", "combine": "bf16_fp32_accumulate",
                   "buffer_sets": nsets},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "dispatch_combine_us": round(dc_time * 1e6, 2),
        "tokens_per_s": round(w.T / dc_time, 1),
        "step_tokens_per_s": round(w.T / (wall / args.steps), 1),
        "roofline": {"kernel": "combine", "bound": "hbm", "achieved": round(comb_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(comb_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "kernels": {s: {k2: (round(v, 4) if isinstance(v, float) else v) for k2, v in d.items()}
                    for s, d in per_kernel.items()},
    }

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, lg_np, x_np, y_np, args.cpu_seconds)

    print(json.dumps(rec), flush=True)
    return 0


def _recorded_traffic(config: str):
    """HBM bytes per combine launch from the committed counter summary, if it
    was taken on the current combine source (else None)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "combine_%s_pmc.txt" % config)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("combine_source_sha") != _kernel_sha():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _kernel_sha() -> str:
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in ("combine.hip", "device.h", "launch.h"):
        with open(os.path.join(root, "combine_group_limited_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(w, lg, x, y, seconds: float):
    """The CPU oracle (plain single-threaded C) on the same batch: route and
    layout once, then FP8 dispatch + combine passes over the whole batch,
    repeated until `seconds` of CPU time have elapsed (at most 8 passes)."""
    import numpy as np

    import oracle

    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    lay = oracle.layout(idx, w.E, w.R)
    q = np.empty((w.nrows, w.H), np.uint8)
    sc = np.empty((w.nrows, w.H // 128), np.float32)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.dispatch_fp8(x, lay["slot"], w.nrows, q, sc)
        oracle.combine(y, lay["slot"], wt)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= seconds or len(times) >= 64:
            break
    t = float(np.median(times))
    return {"value": round((w.bytes_dispatch_fp8() + w.bytes_combine()) / t / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": "full %s batch (%d tokens), FP8 dispatch + combine, median of %d passes, %.2f s each"
                      % (w.name, w.T, len(times), t)}


if __name__ == "__main__":
    sys.exit(main())
