#!/usr/bin/env python3
"""Benchmark of the MoE routing -> FP8 dispatch -> BF16 combine path on one
MI355X.

One step = ep_route_layout (routing and layout) + ep_dispatch (FP8 E4M3,
1x128 scales) + ep_combine over one batch of seeded synthetic input already resident in
HBM (4096 tokens x 7168 hidden, 256 experts in 8 groups, top-4 groups,
top-8 experts, 32 virtual ranks by default).  Expert outputs for the combine
are a resident synthetic buffer (the expert computation is not part of the
path).

Every buffer exists in several copies used round-robin, so that each step
reads its inputs from HBM rather than from the 256 MB Infinity Cache
(--warm-x shares one x between the copies instead, as when the layer before
has just written it, and says so in `config.x`).  The
line also reports the step replayed from a captured HIP graph that holds
one step per buffer set (`graph_step_us`), which removes the host's launch
gaps.

Prints one JSON line.  `ms_per_step` is the wall time of the timed steps,
which hold nothing but the step's own calls.  `value` is dispatch+combine
algorithmic bytes divided by the summed average durations of the dispatch
and combine kernels, from HIP events recorded on the launch stream around
each stage in as many further steps (the buffer sets keep rotating).  The
`roofline` object reports the dominant kernel (combine); `cpu_baseline`
times the CPU oracle on the same batch, on one thread and on every thread
the process may use, and `parity` compares its outputs with the GPU's.

Other workloads (--config), the BF16 payload (--recv-dtype bf16) and the
low-latency path (--path ll: route + dispatch_ll + combine_ll into
fixed-capacity receive rows, decode workload by default; `value` is then the
dispatch+combine time in microseconds) print the same kind of line.

usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config NAME]
                       [--path normal|ll] [--recv-dtype fp8|bf16]
                       [--capacity N] [--sets N] [--no-cpu-baseline] [--warm-x]
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
    ap.add_argument("--config", default=None,
                    help="workload (default: prefill for the normal path, decode for the low-latency path)")
    ap.add_argument("--path", choices=("normal", "ll", "overlap", "dedup"), default="normal",
                    help="normal: route_layout + dispatch + combine; ll: route + dispatch_ll + combine_ll; "
                         "overlap: dispatch + combine on a CU budget next to a bf16 GEMM on the other CUs; "
                         "dedup: per-rank deduplicated dispatch + in-rank partial combine + combine of partials")
    ap.add_argument("--cus", default="16,24,32,64,128", help="CU budgets of the overlap path")
    ap.add_argument("--gemm-n", type=int, default=14336, help="output width of the overlap path's GEMM")
    ap.add_argument("--recv-dtype", choices=("fp8", "bf16"), default="fp8", help="dispatch payload")
    ap.add_argument("--capacity", type=int, default=0, help="low-latency rows per expert (0: T)")
    ap.add_argument("--sets", type=int, default=0,
                    help="copies of all buffers used round-robin (0: enough that every step reads its inputs "
                         "from HBM, not from the caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-x", action="store_true",
                    help="normal path: every buffer set shares one x, which then stays in the Infinity Cache "
                         "(as when the layer before has just written it); the default reads x cold")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="CPU time of the oracle legs (half on one thread, half on all threads)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM counters)")
    ap.add_argument("--ceiling-probe", action="store_true",
                    help="HBM rates of plain kernels (streaming read, write, copy; combine- and dispatch-shaped "
                         "copies without their arithmetic) beside the library's dispatch and combine")
    ap.add_argument("--launch-probe", action="store_true",
                    help="fixed launch costs in the routing, layout and combine launch shapes, and the routing "
                         "kernel's memory pattern without its arithmetic, beside ep_route and ep_route_layout")
    return ap.parse_args()


def buffer_sets(requested: int, touched: int, allocated: int, cached: int) -> int:
    """Copies of the buffers used round-robin, so that every step reads its
    inputs from HBM: at least 4; enough that >= 2 GiB of touched data lies
    between two uses of a copy; and enough that the data a step reads or
    writes through the caches (`cached` bytes per copy: logits, x, scales and
    the index arrays; the streaming (nt) loads and stores of the receive
    rows, y and out do not stay in the 256 MB Infinity Cache) is at least
    twice that cache between two uses of a copy.  Measured on MI355X at
    prefill: with 4 copies part of x was still in the Infinity Cache (FP8
    dispatch 56.4 us; 62.6 us with 8 or 16 copies, 49.8 us with x in the
    cache).  At most 256 copies and 48 GiB allocated."""
    if requested:
        return requested
    n = max(4, -(-(2 << 30) // max(touched, 1)), 1 + -(-(512 << 20) // max(cached, 1)))
    n = min(n, 256, max(4, (48 << 30) // max(allocated, 1)))
    return int(n)


def cached_bytes(w, scale_rows: int) -> int:
    """Bytes per buffer copy that a step moves through the caches: logits,
    x, the FP8 scales of `scale_rows` receive rows and the [T, k] index
    arrays."""
    return w.T * w.E * 4 + w.T * w.H * 2 + scale_rows * (w.H // 128) * 4 + 4 * w.T * w.k * 4


def _copy_gbs(n: int = 1 << 30, reps: int = 5):
    """(microseconds, GB/s read + written) of a plain n-byte device-to-device
    copy, averaged over `reps` copies after one untimed copy."""
    import torch
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.copy_(a)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / reps * 1e-3
    del a, b
    return t * 1e6, 2 * n / t / 1e9


def copy_probe():
    """A plain copy of known size: 5 x 1 GiB device-to-device copies.  Its
    FETCH_SIZE / WRITE_SIZE readings give the factor between those counters
    and bytes actually moved."""
    n = 1 << 30
    us, gbs = _copy_gbs(n)
    print(json.dumps({"kind": "copy_probe", "bytes_read": n, "bytes_written": n,
                      "us": round(us, 1), "gbs_read_plus_write": round(gbs, 1)}), flush=True)
    return 0


def ceiling_probe(args):
    """What plain kernels reach on this GPU (libhbmprobe.so), as ceilings for
    the dispatch and combine kernels: streaming (nt) read, write and copy
    over 1 GiB, the combine's 8:1 read/write mix on sequential streams (1 GiB
    read, 128 MiB written, launched as the combine is), and copies with the combine's access pattern (a 16-byte piece
    of each of a token's k rows gathered into one output piece) and the FP8
    dispatch's payload pattern (a token's bf16 row stored to k rows of H
    bytes), at the prefill shape, on the canonical layout's receive rows and
    on sequential rows (t*k + j), beside ep_combine and ep_dispatch on the
    same rows.  Each probe rotates over copies of its buffers, so that every
    run reads from HBM: two of the 1 GiB buffers and of y (streamed with nt
    loads), and 12 of x (700 MB, read through the caches: with two copies x
    stays in the 256 MB Infinity Cache).  HIP events around `steps` runs."""
    import numpy as np
    import torch

    import combine_group_limited_amd as ep
    from combine_group_limited_amd import _lib as L
    from combine_group_limited_amd import build as B
    import workloads as W

    if not os.path.exists(B.PROBE_LIB_PATH):
        B.build()
    P = ctypes.CDLL(B.PROBE_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    P.hbm_probe_read.argtypes = [vp, sz, vp, vp]
    P.hbm_probe_write.argtypes = [vp, sz, vp]
    P.hbm_probe_copy.argtypes = [vp, vp, sz, vp]
    P.hbm_probe_mix8.argtypes = [vp, vp, sz, vp]
    P.hbm_probe_gather.argtypes = [vp, vp, vp, i, i, i, i, vp]
    P.hbm_probe_scatter.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib = L.lib()
    dev = torch.device("cuda", 0)
    sh = int(torch.cuda.current_stream().cuda_stream)
    w = W.PREFILL
    cfg = ep.Config.of(w)
    c = cfg.c()
    cp = ctypes.byref(c)
    GiB = 1 << 30
    big = [torch.empty(GiB, dtype=torch.uint8, device=dev) for _ in range(4)]
    for t in big:
        t.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    lay = ep.route_layout(cfg, torch.from_numpy(W.gen_logits(w)).to(dev))
    slot = lay["slot"]
    seq = torch.arange(w.nrows, dtype=torch.int32, device=dev).view(w.T, w.k)
    y = [torch.from_numpy(W.gen_y(w).view(np.int16)).view(torch.bfloat16).to(dev) for _ in range(2)]
    x0 = torch.from_numpy(W.gen_x(w).view(np.int16)).view(torch.bfloat16).to(dev)
    NX = 12
    x = [x0] + [x0.clone() for _ in range(NX - 1)]
    out = [torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    recv = [torch.empty((w.nrows, w.H), dtype=torch.uint8, device=dev) for _ in range(2)]
    sc = [torch.empty((w.nrows, w.H // 128), dtype=torch.float32, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    hev = HipEvents()
    n = max(args.steps, 2)

    def timed(fn):
        for j in range(2):
            if fn(j) != 0:
                raise RuntimeError("probe launch failed")
        e = hev.create(2)
        hev.record(e[0], sh)
        for j in range(n):
            fn(j)
        hev.record(e[1], sh)
        t = hev.seconds(e[0], e[1]) / n
        hev.destroy(e)
        return t

    gather_b = w.T * (2 * w.k * w.H + 2 * w.H + 4 * w.k)
    scatter_b = w.T * (2 * w.H + w.k * w.H + 4 * w.k)
    probes = {
        "read_1GiB": (GiB, lambda j: P.hbm_probe_read(big[j % 2].data_ptr(), GiB, sink.data_ptr(), sh)),
        "write_1GiB": (GiB, lambda j: P.hbm_probe_write(big[j % 2].data_ptr(), GiB, sh)),
        "copy_1GiB": (2 * GiB, lambda j: P.hbm_probe_copy(big[j % 2].data_ptr(), big[2 + j % 2].data_ptr(), GiB, sh)),
        "mix8to1_1GiB": (GiB + GiB // 8, lambda j: P.hbm_probe_mix8(big[j % 2].data_ptr(), big[2 + j % 2].data_ptr(),
                                                                    GiB // 8, sh)),
        "gather_layout_rows": (gather_b, lambda j: P.hbm_probe_gather(y[j % 2].data_ptr(), slot.data_ptr(),
                                                                      out[j % 2].data_ptr(), w.T, w.H, w.k, w.nrows, sh)),
        "gather_sequential_rows": (gather_b, lambda j: P.hbm_probe_gather(y[j % 2].data_ptr(), seq.data_ptr(),
                                                                          out[j % 2].data_ptr(), w.T, w.H, w.k,
                                                                          w.nrows, sh)),
        "combine_layout_rows": (w.bytes_combine(), lambda j: lib.ep_combine(cp, y[j % 2].data_ptr(), slot.data_ptr(),
                                                                           lay["w"].data_ptr(), out[j % 2].data_ptr(),
                                                                           sh)),
        "scatter_layout_rows": (scatter_b, lambda j: P.hbm_probe_scatter(x[j % NX].data_ptr(), slot.data_ptr(),
                                                                         recv[j % 2].data_ptr(), w.T, w.H, w.k,
                                                                         w.nrows, sh)),
        "scatter_sequential_rows": (scatter_b, lambda j: P.hbm_probe_scatter(x[j % NX].data_ptr(), seq.data_ptr(),
                                                                             recv[j % 2].data_ptr(), w.T, w.H, w.k,
                                                                             w.nrows, sh)),
        "dispatch_fp8_layout_rows": (w.bytes_dispatch_fp8(),
                                     lambda j: lib.ep_dispatch(cp, x[j % NX].data_ptr(), slot.data_ptr(),
                                                               L.EP_RECV_FP8_E4M3, recv[j % 2].data_ptr(),
                                                               sc[j % 2].data_ptr(), sh)),
    }
    res = {}
    for name, (nbytes, fn) in probes.items():
        t = timed(fn)
        res[name] = {"us": round(t * 1e6, 2), "bytes": nbytes, "gbs": round(nbytes / t / 1e9, 1),
                     "frac_of_8000": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        print("probe %-26s %9.2f us %8.1f GB/s" % (name, t * 1e6, nbytes / t / 1e9), file=sys.stderr, flush=True)
    print(json.dumps({"metric": "HBM ceiling probes (plain kernels) beside dispatch and combine, prefill shape",
                      "unit": "GB/s", "peak": HBM_PEAK_GBS, "steps": n,
                      "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "topk": w.k},
                      "probes": res}), flush=True)
    return 0


def launch_probe(args):
    """Fixed costs beside the routing and layout kernels (libhbmprobe.so): a
    launch that does nothing, in the shapes of the routing launch with column
    counts (256 workgroups of 1024 threads, 8 KiB of LDS), of the routing
    launch without them (1024 of 256), of the layout's assign launch (64 of
    512, its 42 KiB of LDS) and of the combine (57344 one-wave workgroups);
    the routing kernel's memory pattern without its arithmetic (one wavefront
    per token reads the token's 256 fp32 logits and writes 8 words to each
    of two [T, k] outputs) at 16 and 4 tokens per workgroup; and beside them
    ep_route and ep_route_layout, at the prefill shape.  A 512 MiB fill
    through the caches before each launch puts the logits back in HBM.  HIP
    events around each launch; the median over `steps` launches."""
    import torch

    import combine_group_limited_amd as ep
    from combine_group_limited_amd import _lib as L
    from combine_group_limited_amd import build as B
    import workloads as W

    if not os.path.exists(B.PROBE_LIB_PATH):
        B.build()
    P = ctypes.CDLL(B.PROBE_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    P.hbm_probe_empty.argtypes = [i, i, sz, vp]
    P.hbm_probe_token_rows.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib = L.lib()
    dev = torch.device("cuda", 0)
    sh = int(torch.cuda.current_stream().cuda_stream)
    w = W.PREFILL
    cfg = ep.Config.of(w)
    c = cfg.c()
    cp = ctypes.byref(c)
    lg = torch.from_numpy(W.gen_logits(w)).to(dev)
    o = ep.route_layout(cfg, lg)
    ws = o["workspace"]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    o1 = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    o2 = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    hev = HipEvents()
    n = max(args.steps, 3)
    assign_lds = (12 * 8 + 4) * w.E + 2 * 8 * w.E * 4 + 4 * w.R
    probes = {
        "empty_256x1024_8KiB": lambda: P.hbm_probe_empty(256, 1024, 8192, sh),
        "empty_1024x256": lambda: P.hbm_probe_empty(1024, 256, 0, sh),
        "empty_64x512_%dB" % assign_lds: lambda: P.hbm_probe_empty(64, 512, assign_lds, sh),
        "empty_57344x64": lambda: P.hbm_probe_empty(57344, 64, 0, sh),
        "token_rows_16_per_wg": lambda: P.hbm_probe_token_rows(lg.data_ptr(), o1.data_ptr(), o2.data_ptr(), w.T, w.E,
                                                               w.k, 16, sh),
        "token_rows_4_per_wg": lambda: P.hbm_probe_token_rows(lg.data_ptr(), o1.data_ptr(), o2.data_ptr(), w.T, w.E,
                                                              w.k, 4, sh),
        "ep_route": lambda: lib.ep_route(cp, lg.data_ptr(), o["idx"].data_ptr(), o["w"].data_ptr(), sh),
        "ep_route_layout": lambda: lib.ep_route_layout(cp, lg.data_ptr(), o["idx"].data_ptr(), o["w"].data_ptr(),
                                                       o["cnt"].data_ptr(), o["ntok_rank"].data_ptr(),
                                                       o["off"].data_ptr(), o["slot"].data_ptr(),
                                                       o["recv_token"].data_ptr(), ws.data_ptr(), ws.numel(), sh),
    }
    res = {}
    for name, fn in probes.items():
        if fn() != 0:
            raise RuntimeError("probe %s failed" % name)
        ts = []
        for j in range(n):
            flush.fill_(j & 0xFF)
            e = hev.create(2)
            hev.record(e[0], sh)
            fn()
            hev.record(e[1], sh)
            ts.append(hev.seconds(e[0], e[1]))
            hev.destroy(e)
        ts.sort()
        res[name] = {"median_us": round(ts[len(ts) // 2] * 1e6, 2), "p10_us": round(ts[len(ts) // 10] * 1e6, 2)}
        print("probe %-28s %7.2f us" % (name, ts[len(ts) // 2] * 1e6), file=sys.stderr, flush=True)
    print(json.dumps({"metric": "launch floors and the routing kernel's memory pattern beside routing and layout",
                      "unit": "us", "steps": n,
                      "config": {"workload": w.name, "tokens": w.T, "experts": w.E, "topk": w.k},
                      "probes": res}), flush=True)
    return 0


HEADLINE_METRIC = "dispatch+combine HBM GB/s and % of peak at 4096 tok x 7168 hidden top-8"


def timed_steps(args, nsets, launch_stages, stages):
    """Runs `warmup` untimed steps, then `steps` timed steps with nothing
    inside them but the step's own calls (the wall clock between two
    synchronisations gives the step time), then `steps` more in which
    launch_stages(set_index, record) records an event before each stage and
    one after the last (the per-stage durations).  The buffer sets rotate
    through all three runs.  Returns (per-stage durations in seconds, wall
    seconds of the timed steps)."""
    import torch
    hev = HipEvents()
    sh = int(torch.cuda.current_stream().cuda_stream)
    n = len(stages) + 1
    warm = [hev.create(n) for _ in range(max(args.warmup, 0))]
    for i, ev in enumerate(warm):
        launch_stages(i % nsets, lambda q, ev=ev: hev.record(ev[q], sh))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        launch_stages((args.warmup + i) % nsets, lambda q: None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [hev.create(n) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, ev in enumerate(evs):
        launch_stages((args.warmup + args.steps + i) % nsets, lambda q, ev=ev: hev.record(ev[q], sh))
    torch.cuda.synchronize()
    dur = {s: [hev.seconds(ev[i], ev[i + 1]) for ev in evs] for i, s in enumerate(stages)}
    for ev in warm + evs:
        hev.destroy(ev)
    return dur, wall


def launch_step(lib, cp, p, code, ws, nws, sh, check):
    """One step of the normal path on stream handle `sh`, no events."""
    check(lib.ep_route_layout(cp, p["logits"], p["idx"], p["wt"], p["cnt"], p["ntok"], p["off"], p["slot"],
                              p["recv_token"], ws.data_ptr(), nws, sh), "ep_route_layout")
    check(lib.ep_dispatch(cp, p["x"], p["slot"], code, p["recv"], p["scales"], sh), "ep_dispatch")
    check(lib.ep_combine(cp, p["y"], p["slot"], p["wt"], p["out"], sh), "ep_combine")


def graph_step_us(args, nsets, step_on):
    """Average time of one step replayed from a captured HIP graph.  One
    graph holds at least 8 steps, cycling through the buffer sets (a whole
    number of cycles), so the graph's own launch cost is spread over them,
    as when a loop of steps is captured; events around all replays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_on(0, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    per_graph = nsets * -(-8 // nsets)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            step_on(i % nsets, torch.cuda.current_stream().cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-max(args.steps, 1) // per_graph))
    hev = HipEvents()
    e = hev.create(2)
    sh = int(torch.cuda.current_stream().cuda_stream)
    hev.record(e[0], sh)
    for _ in range(reps):
        g.replay()
    hev.record(e[1], sh)
    t = hev.seconds(e[0], e[1]) / (reps * per_graph)
    hev.destroy(e)
    del g
    return t * 1e6


def kernel_table(dur, bytes_):
    import numpy as np
    out = {}
    for s, v in dur.items():
        avg = float(np.mean(v))
        out[s] = {"avg_us": round(avg * 1e6, 4), "median_us": round(float(np.median(v)) * 1e6, 4),
                  "p10_us": round(float(np.percentile(v, 10)) * 1e6, 4),
                  "p90_us": round(float(np.percentile(v, 90)) * 1e6, 4),
                  "algorithmic_bytes": bytes_[s], "gbs": round(bytes_[s] / avg / 1e9, 4),
                  "frac": round(bytes_[s] / avg / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def run_normal(args, w):
    """route_layout (routing and layout) + dispatch + combine on resident buffers."""
    import numpy as np
    import torch

    import combine_group_limited_amd as ep
    from combine_group_limited_amd import _lib as L
    import workloads as W

    cfg = ep.Config.of(w)
    dev = torch.device("cuda", 0)
    fp8 = args.recv_dtype == "fp8"
    bytes_ = dict(route_layout=w.bytes_route() + w.bytes_layout(),
                  dispatch=w.bytes_dispatch_fp8() if fp8 else w.bytes_dispatch_bf16(), combine=w.bytes_combine())
    touched = sum(bytes_.values())
    nsets = buffer_sets(args.sets, touched, touched, cached_bytes(w, w.nrows if fp8 else 0))

    # Resident inputs and outputs, in `nsets` copies used round-robin so that
    # no step finds its data in the 256 MB Infinity Cache or the L2s.
    lg_np, x_np, y_np = W.gen_logits(w), W.gen_x(w), W.gen_y(w)
    logits0 = torch.from_numpy(lg_np).to(dev)
    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    y0 = torch.from_numpy(y_np.view(np.int16)).view(torch.bfloat16).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    ws = torch.empty(max(16, ep.route_layout_workspace_bytes(cfg)), dtype=torch.uint8, device=dev)
    sets = []
    for i in range(nsets):
        sets.append(dict(
            logits=logits0 if i == 0 else logits0.clone(),
            x=x0 if i == 0 or args.warm_x else x0.clone(),
            y=y0 if i == 0 else y0.clone(),
            idx=torch.empty((w.T, w.k), **i32),
            wt=torch.empty((w.T, w.k), dtype=torch.float32, device=dev),
            cnt=torch.empty(w.E, **i32), ntok=torch.empty(w.R, **i32), off=torch.empty(w.E + 1, **i32),
            slot=torch.empty((w.T, w.k), **i32), recv_token=torch.empty(w.nrows, **i32),
            recv=torch.empty((w.nrows, w.H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            scales=torch.empty((w.nrows, w.H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)))

    # validate once through the checked binding, then call the C ABI directly
    for b in sets:
        ep.route_layout(cfg, b["logits"], dict(idx=b["idx"], w=b["wt"], cnt=b["cnt"], ntok_rank=b["ntok"],
                                               off=b["off"], slot=b["slot"], recv_token=b["recv_token"]), ws)
        ep.dispatch(cfg, b["x"], b["slot"], args.recv_dtype, b["recv"], b["scales"])
        ep.combine(cfg, b["y"], b["slot"], b["wt"], b["out"])
    torch.cuda.synchronize()
    ptr = [{k: (v.data_ptr() if v is not None else None) for k, v in b.items()} for b in sets]
    lib = L.lib()
    c = cfg.c()
    cp = ctypes.byref(c)
    sh = int(torch.cuda.current_stream().cuda_stream)
    code = L.EP_RECV_FP8_E4M3 if fp8 else L.EP_RECV_BF16
    nws = ws.numel()

    def check(rc, name):
        if rc != 0:
            raise RuntimeError("%s failed: %s" % (name, lib.ep_strerror(rc).decode()))

    def launch(i, rec):
        p = ptr[i]
        rec(0)
        check(lib.ep_route_layout(cp, p["logits"], p["idx"], p["wt"], p["cnt"], p["ntok"], p["off"], p["slot"],
                                  p["recv_token"], ws.data_ptr(), nws, sh), "ep_route_layout")
        rec(1)
        check(lib.ep_dispatch(cp, p["x"], p["slot"], code, p["recv"], p["scales"], sh), "ep_dispatch")
        rec(2)
        check(lib.ep_combine(cp, p["y"], p["slot"], p["wt"], p["out"], sh), "ep_combine")
        rec(3)

    stages = ("route_layout", "dispatch", "combine")
    dur, wall = timed_steps(args, nsets, launch, stages)
    kt = kernel_table(dur, bytes_)
    graph_us = graph_step_us(args, nsets, lambda i, sh: launch_step(lib, cp, ptr[i], code, ws, nws, sh, check))
    avg = {s: kt[s]["avg_us"] * 1e-6 for s in stages}
    dc_bytes = bytes_["dispatch"] + bytes_["combine"]
    dc_time = avg["dispatch"] + avg["combine"]
    value = dc_bytes / dc_time / 1e9
    headline = w.name == "prefill" and fp8
    comb_gbs = bytes_["combine"] / avg["combine"] / 1e9
    rec = {
        "metric": HEADLINE_METRIC if headline else
        "dispatch+combine HBM GB/s and %% of peak at %d tok x %d hidden top-%d (%s dispatch)" % (
            w.T, w.H, w.k, args.recv_dtype.upper()),
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
        "storage_dtypes": {"dispatch": "fp8_e4m3 codes + fp32 scales" if fp8 else "bf16", "combine": "bf16"},
        "data": "synthetic",
        "config": {"workload": w.name, "path": "normal", "tokens": w.T, "hidden": w.H, "experts": w.E,
                   "groups": w.G, "topk_groups": w.TG, "topk": w.k, "virtual_ranks": w.R,
                   "dispatch": "fp8_e4m3_1x128_fp32_scales" if fp8 else "bf16",
                   "combine": "bf16_fp32_accumulate", "buffer_sets": nsets,
                   "x": "one copy shared by every buffer set (warm)" if args.warm_x else "own copy per buffer set"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "dispatch_combine_us": round(dc_time * 1e6, 2),
        "tokens_per_s": round(w.T / dc_time, 1),
        "step_tokens_per_s": round(w.T / (wall / args.steps), 1),
        "graph_step_us": round(graph_us, 2),
        "graph_step_tokens_per_s": round(w.T / (graph_us * 1e-6), 1),
        "context": {"device_copy_gbs": round(_copy_gbs()[1], 1),
                    "note": "plain 1 GiB device-to-device copy, bytes read + written per second: "
                            "a practical ceiling beside the 8000 GB/s peak"},
        "roofline": {"kernel": "combine", "bound": "hbm", "achieved": round(comb_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(comb_gbs / HBM_PEAK_GBS, 4),
                     "traffic": _recorded_traffic("combine", w.name)},
        "kernels": kt,
    }
    dkey = "dispatch_fp8" if fp8 else "dispatch_bf16"
    rec["kernels"]["dispatch"]["traffic"] = _recorded_traffic(dkey, w.name)
    rec["inputs"] = provenance(w, {"logits": lg_np, "x": x_np, "y": y_np})
    if not args.no_cpu_baseline:
        def to_host(t):
            t = t.detach().cpu()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

        gpu = {k: to_host(v) for k, v in sets[0].items()
               if v is not None and k in ("idx", "wt", "cnt", "ntok", "off", "slot", "recv_token", "recv",
                                          "scales", "out")}
        rec["parity"], _, wt_o, lay_o = oracle_parity(w, fp8, gpu, lg_np, x_np, y_np)
        del gpu
        rec["cpu_baseline"] = cpu_baseline(w, fp8, x_np, y_np, wt_o, lay_o, args.cpu_seconds)
    return rec


def run_ll(args, w):
    """route + dispatch_ll + combine_ll (fixed-capacity receive rows) on
    resident buffers."""
    import numpy as np
    import torch

    import combine_group_limited_amd as ep
    from combine_group_limited_amd import _lib as L
    import workloads as W

    cfg = ep.Config.of(w)
    dev = torch.device("cuda", 0)
    fp8 = args.recv_dtype == "fp8"
    cap = args.capacity or w.T
    nrows = w.E * cap
    bytes_ = dict(route=w.bytes_route(),
                  dispatch_ll=(w.bytes_dispatch_fp8() if fp8 else w.bytes_dispatch_bf16()),
                  combine_ll=w.bytes_combine())
    touched = sum(bytes_.values())
    allocated = nrows * w.H * (1 if fp8 else 2) + nrows * w.H * 2 + touched
    nsets = buffer_sets(args.sets, touched, allocated, cached_bytes(w, nrows if fp8 else 0))

    lg_np, x_np = W.gen_logits(w), W.gen_x(w)
    logits0 = torch.from_numpy(lg_np).to(dev)
    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    y0 = torch.randn((nrows, w.H), device=dev).to(torch.bfloat16)   # expert outputs, any values
    i32 = dict(dtype=torch.int32, device=dev)
    sets = []
    for i in range(nsets):
        sets.append(dict(
            logits=logits0 if i == 0 else logits0.clone(),
            x=x0 if i == 0 or args.warm_x else x0.clone(),
            y=y0 if i == 0 else y0.clone(),
            idx=torch.empty((w.T, w.k), **i32),
            wt=torch.empty((w.T, w.k), dtype=torch.float32, device=dev),
            count=torch.empty(w.E, **i32), src=torch.empty(nrows, **i32), slot=torch.empty((w.T, w.k), **i32),
            recv=torch.empty((nrows, w.H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            scales=torch.empty((nrows, w.H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)))
    for b in sets:
        ep.route(cfg, b["logits"], b["idx"], b["wt"])
        ep.dispatch_ll(cfg, b["x"], b["idx"], cap, args.recv_dtype, b["recv"], b["scales"], b["count"], b["src"],
                       b["slot"])
        ep.combine_ll(cfg, cap, b["y"], b["slot"], b["wt"], b["out"])
    torch.cuda.synchronize()
    ptr = [{k: (v.data_ptr() if v is not None else None) for k, v in b.items()} for b in sets]
    lib = L.lib()
    c = cfg.c()
    cp = ctypes.byref(c)
    sh = int(torch.cuda.current_stream().cuda_stream)
    code = L.EP_RECV_FP8_E4M3 if fp8 else L.EP_RECV_BF16

    def check(rc, name):
        if rc != 0:
            raise RuntimeError("%s failed: %s" % (name, lib.ep_strerror(rc).decode()))

    def launch(i, rec, st=sh):
        p = ptr[i]
        rec(0)
        check(lib.ep_route(cp, p["logits"], p["idx"], p["wt"], st), "ep_route")
        rec(1)
        check(lib.ep_dispatch_ll(cp, p["x"], p["idx"], cap, code, p["recv"], p["scales"], p["count"], p["src"],
                                 p["slot"], st), "ep_dispatch_ll")
        rec(2)
        check(lib.ep_combine_ll(cp, cap, p["y"], p["slot"], p["wt"], p["out"], st), "ep_combine_ll")
        rec(3)

    stages = ("route", "dispatch_ll", "combine_ll")
    dur, wall = timed_steps(args, nsets, launch, stages)
    graph_us = graph_step_us(args, nsets, lambda i, st: launch(i, lambda q: None, int(st)))
    kt = kernel_table(dur, bytes_)
    avg = {s: kt[s]["avg_us"] * 1e-6 for s in stages}
    dc_time = avg["dispatch_ll"] + avg["combine_ll"]
    dc_bytes = bytes_["dispatch_ll"] + bytes_["combine_ll"]
    comb_gbs = bytes_["combine_ll"] / avg["combine_ll"] / 1e9
    rec = {
        "metric": "low-latency dispatch+combine time at %d tok x %d hidden top-%d (%s dispatch)" % (
            w.T, w.H, w.k, args.recv_dtype.upper()),
        "value": round(dc_time * 1e6, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "path": "low_latency", "tokens": w.T, "hidden": w.H, "experts": w.E,
                   "groups": w.G, "topk_groups": w.TG, "topk": w.k, "capacity": cap,
                   "dispatch": "fp8_e4m3_1x128_fp32_scales" if fp8 else "bf16",
                   "combine": "bf16_fp32_accumulate", "buffer_sets": nsets},
        "dispatch_combine_gbs": round(dc_bytes / dc_time / 1e9, 1),
        "step_us": round(sum(avg.values()) * 1e6, 2),
        "graph_step_us": round(graph_us, 2),
        "roofline": {"kernel": "combine_ll", "bound": "hbm", "achieved": round(comb_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(comb_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "kernels": kt,
    }
    return rec


def run_overlap(args, w):
    """Dispatch + combine confined to CUs [0, N) (ep_stream_create_cu_range)
    while a stand-in compute stream runs bf16 GEMMs (hipBLASLt through
    torch.matmul, [T, H] x [H, gemm_n], by default an expert up-projection of
    width 2 x 7168) on CUs [N, all): each alone, then both at once, for each
    budget N."""
    import numpy as np
    import torch

    import combine_group_limited_amd as ep
    from combine_group_limited_amd import _lib as L
    import workloads as W

    cfg = ep.Config.of(w)
    dev = torch.device("cuda", 0)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    dc_bytes = w.bytes_dispatch_fp8() + w.bytes_combine()
    nsets = buffer_sets(args.sets, dc_bytes, dc_bytes, cached_bytes(w, w.nrows))
    lg = torch.from_numpy(W.gen_logits(w)).to(dev)
    idx, wt = ep.route(cfg, lg)
    slot = ep.get_layout(cfg, idx)["slot"]
    x0 = torch.from_numpy(W.gen_x(w).view(np.int16)).view(torch.bfloat16).to(dev)
    y0 = torch.from_numpy(W.gen_y(w).view(np.int16)).view(torch.bfloat16).to(dev)
    sets = [dict(x=x0 if i == 0 else x0.clone(), y=y0 if i == 0 else y0.clone(),
                 recv=torch.empty((w.nrows, w.H), dtype=torch.uint8, device=dev),
                 scales=torch.empty((w.nrows, w.H // 128), dtype=torch.float32, device=dev),
                 out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)) for i in range(nsets)]
    gn = args.gemm_n
    A = torch.randn((w.T, w.H), device=dev).to(torch.bfloat16)
    B = torch.randn((w.H, gn), device=dev).to(torch.bfloat16)
    C = torch.empty((w.T, gn), dtype=torch.bfloat16, device=dev)
    gemm_flop = 2.0 * w.T * w.H * gn
    lib = L.lib()
    c = cfg.c()
    cp = ctypes.byref(c)
    ptr = [{k: v.data_ptr() for k, v in b.items()} for b in sets]
    torch.cuda.synchronize()

    def dc(i, sh):
        p = ptr[i % nsets]
        if lib.ep_dispatch(cp, p["x"], slot.data_ptr(), L.EP_RECV_FP8_E4M3, p["recv"], p["scales"], sh) != 0:
            raise RuntimeError("ep_dispatch failed")
        if lib.ep_combine(cp, p["y"], slot.data_ptr(), wt.data_ptr(), p["out"], sh) != 0:
            raise RuntimeError("ep_combine failed")

    def gemm(i, sh):
        torch.matmul(A, B, out=C)

    hev = HipEvents()
    n = max(args.steps, 1)

    def alone(stream, fn):
        sh = stream.cuda_stream
        with torch.cuda.stream(stream.torch):
            for i in range(max(args.warmup, 1)):
                fn(i, sh)
            torch.cuda.synchronize()
            e = hev.create(2)
            hev.record(e[0], sh)
            for i in range(n):
                fn(i, sh)
            hev.record(e[1], sh)
            t = hev.seconds(e[0], e[1]) / n
            hev.destroy(e)
        return t

    def together(sc, sg):
        e = hev.create(4)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hev.record(e[0], sc.cuda_stream)
        hev.record(e[2], sg.cuda_stream)
        for i in range(n):  # interleave the issue so both queues stay fed
            with torch.cuda.stream(sg.torch):
                gemm(i, sg.cuda_stream)
            dc(i, sc.cuda_stream)
        hev.record(e[1], sc.cuda_stream)
        hev.record(e[3], sg.cuda_stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / n
        r = hev.seconds(e[0], e[1]) / n, hev.seconds(e[2], e[3]) / n, wall
        hev.destroy(e)
        return r

    with ep.CuRangeStream(0, ncu) as full:
        dc_full, gemm_full = alone(full, dc), alone(full, gemm)
    rows = []
    for N in [int(v) for v in args.cus.split(",") if v.strip()]:
        if not 0 < N < ncu:
            continue
        with ep.CuRangeStream(0, N) as sc, ep.CuRangeStream(N, ncu - N) as sg:
            dca, ga = alone(sc, dc), alone(sg, gemm)
            dco, go, wall = together(sc, sg)
        rows.append({"comm_cus": N, "compute_cus": ncu - N,
                     "dc_alone_us": round(dca * 1e6, 2), "gemm_alone_us": round(ga * 1e6, 2),
                     "dc_overlapped_us": round(dco * 1e6, 2), "gemm_overlapped_us": round(go * 1e6, 2),
                     "wall_per_pair_us": round(wall * 1e6, 2),
                     "dc_overlapped_gbs": round(dc_bytes / dco / 1e9, 1),
                     "gemm_overlapped_tflops": round(gemm_flop / go / 1e12, 1),
                     "serial_full_gpu_us": round((dc_full + gemm_full) * 1e6, 2)})
    return {
        "metric": "dispatch+combine on a CU budget overlapped with a bf16 GEMM on the other CUs",
        "value": None if not rows else min(r["wall_per_pair_us"] for r in rows),
        "unit": "us per (dispatch+combine, GEMM) pair, best budget",
        "n_gpus": 1, "steps": n, "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": w.name, "path": "overlap", "tokens": w.T, "hidden": w.H, "topk": w.k,
                   "gemm": "bf16 [%d, %d] x [%d, %d] (torch.matmul)" % (w.T, w.H, w.H, gn), "cus": ncu,
                   "buffer_sets": nsets},
        "full_gpu": {"dc_us": round(dc_full * 1e6, 2), "gemm_us": round(gemm_full * 1e6, 2),
                     "gemm_tflops": round(gemm_flop / gemm_full / 1e12, 1)},
        "budgets": rows,
    }


def run_dedup(args, w):
    """route_layout + rank layout + deduplicated FP8 dispatch (one row per
    (token, rank)) + in-rank partial combine + combine of the partial rows,
    on resident buffers."""
    import numpy as np
    import torch

    import combine_group_limited_amd as ep
    from combine_group_limited_amd import _lib as L
    import workloads as W

    cfg = ep.Config.of(w)
    dev = torch.device("cuda", 0)
    lg_np, x_np, y_np = W.gen_logits(w), W.gen_x(w), W.gen_y(w)
    B = w.H // 128
    P = w.T * w.k
    logits0 = torch.from_numpy(lg_np).to(dev)
    # rank rows of the seeded routing (the byte model depends on them), from
    # the library's own rank layout
    c_idx, _ = ep.route(cfg, logits0)
    rows = int(ep.get_rank_layout(cfg, c_idx, with_rank_token=False)["rank_offset"][-1].item())
    bytes_ = dict(route_layout=w.bytes_route() + w.bytes_layout(),
                  rank_layout=P * 8 + 4 * (2 * w.R + 1),
                  dispatch=w.T * 2 * w.H + rows * (w.H + 4 * B) + 4 * P,
                  partial=2 * w.H * P + 2 * w.H * rows + 16 * P,
                  combine_ranks=2 * w.H * rows + 2 * w.H * w.T + 4 * P)
    touched = sum(bytes_.values())
    nsets = buffer_sets(args.sets, touched, touched, cached_bytes(w, rows))
    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    y0 = torch.from_numpy(y_np.view(np.int16)).view(torch.bfloat16).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    ws = torch.empty(max(256, ep.route_layout_workspace_bytes(cfg)), dtype=torch.uint8, device=dev)
    rws = torch.empty(max(256, ep.rank_layout_workspace_bytes(cfg)), dtype=torch.uint8, device=dev)
    sets = []
    for i in range(nsets):
        sets.append(dict(
            logits=logits0 if i == 0 else logits0.clone(), x=x0 if i == 0 else x0.clone(),
            y=y0 if i == 0 else y0.clone(),
            idx=torch.empty((w.T, w.k), **i32), wt=torch.empty((w.T, w.k), dtype=torch.float32, device=dev),
            cnt=torch.empty(w.E, **i32), ntok=torch.empty(w.R, **i32), off=torch.empty(w.E + 1, **i32),
            slot=torch.empty((w.T, w.k), **i32),
            rcnt=torch.empty(w.R, **i32), roff=torch.empty(w.R + 1, **i32), rslot=torch.empty((w.T, w.k), **i32),
            recv=torch.empty((P, w.H), dtype=torch.uint8, device=dev),
            scales=torch.empty((P, B), dtype=torch.float32, device=dev),
            partial=torch.empty((P, w.H), dtype=torch.bfloat16, device=dev),
            out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)))
    for b in sets:
        ep.route_layout(cfg, b["logits"], dict(idx=b["idx"], w=b["wt"], cnt=b["cnt"], ntok_rank=b["ntok"],
                                               off=b["off"], slot=b["slot"]), ws, with_recv_token=False)
        ep.get_rank_layout(cfg, b["idx"], dict(rank_count=b["rcnt"], rank_offset=b["roff"], rank_slot=b["rslot"]),
                           rws, with_rank_token=False)
        ep.dispatch(cfg, b["x"], b["rslot"], "fp8", b["recv"], b["scales"])
        ep.combine_rank_partial(cfg, b["y"], b["idx"], b["slot"], b["wt"], b["rslot"], b["partial"])
        ep.combine_ranks(cfg, b["partial"], b["rslot"], b["out"])
    torch.cuda.synchronize()
    assert int(sets[0]["roff"][-1]) == rows
    ptr = [{k: v.data_ptr() for k, v in b.items()} for b in sets]
    lib = L.lib()
    c = cfg.c()
    cp = ctypes.byref(c)
    sh = int(torch.cuda.current_stream().cuda_stream)

    def check(rc, name):
        if rc != 0:
            raise RuntimeError("%s failed: %s" % (name, lib.ep_strerror(rc).decode()))

    def launch(i, rec):
        p = ptr[i]
        rec(0)
        check(lib.ep_route_layout(cp, p["logits"], p["idx"], p["wt"], p["cnt"], p["ntok"], p["off"], p["slot"], None,
                                  ws.data_ptr(), ws.numel(), sh), "ep_route_layout")
        rec(1)
        check(lib.ep_get_rank_layout(cp, p["idx"], p["rcnt"], p["roff"], p["rslot"], None, rws.data_ptr(),
                                     rws.numel(), sh), "ep_get_rank_layout")
        rec(2)
        check(lib.ep_dispatch(cp, p["x"], p["rslot"], L.EP_RECV_FP8_E4M3, p["recv"], p["scales"], sh), "ep_dispatch")
        rec(3)
        check(lib.ep_combine_rank_partial(cp, p["y"], p["idx"], p["slot"], p["wt"], p["rslot"], p["partial"], sh),
              "ep_combine_rank_partial")
        rec(4)
        check(lib.ep_combine_ranks(cp, p["partial"], p["rslot"], p["out"], sh), "ep_combine_ranks")
        rec(5)

    stages = ("route_layout", "rank_layout", "dispatch", "partial", "combine_ranks")
    dur, wall = timed_steps(args, nsets, launch, stages)
    kt = kernel_table(dur, bytes_)
    avg = {s: kt[s]["avg_us"] * 1e-6 for s in stages}
    moved = bytes_["dispatch"] + bytes_["partial"] + bytes_["combine_ranks"]
    t_dc = avg["dispatch"] + avg["partial"] + avg["combine_ranks"]
    # bytes that would cross links between GPUs: payload + scales out, one
    # bf16 row per (token, rank) back, against one row per (token, expert)
    link_dedup = rows * (w.H + 4 * B + 2 * w.H)
    link_flat = P * (w.H + 4 * B + 2 * w.H)
    return {
        "metric": "deduplicated dispatch + two-level combine HBM GB/s at %d tok x %d hidden top-%d" % (w.T, w.H, w.k),
        "value": round(moved / t_dc / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": w.name, "path": "dedup", "tokens": w.T, "hidden": w.H, "experts": w.E,
                   "topk": w.k, "virtual_ranks": w.R, "buffer_sets": nsets},
        "rank_rows": rows, "rank_rows_per_token": round(rows / w.T, 3),
        "dedup_dispatch_combine_us": round(t_dc * 1e6, 2),
        "link_bytes": {"flat": link_flat, "dedup": link_dedup, "saved_frac": round(1 - link_dedup / link_flat, 4)},
        "kernels": kt,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU exchange "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2
    if args.warm_x and args.path != "normal":
        print("--warm-x applies to the normal path only (--path %s requested)" % args.path, file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe()
    if args.ceiling_probe:
        return ceiling_probe(args)
    if args.launch_probe:
        return launch_probe(args)

    import torch
    import workloads as W

    name = args.config or ("decode" if args.path == "ll" else "prefill")
    w = W.CONFIGS[name]
    torch.cuda.set_device(0)
    runner = {"normal": run_normal, "ll": run_ll, "overlap": run_overlap, "dedup": run_dedup}[args.path]
    rec = runner(args, w)
    print(json.dumps(rec), flush=True)
    return 0


def _recorded_traffic(kernel: str, config: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    for `config`, if it was taken on the kernel's current source (else
    None)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "%s_%s_pmc.txt" % (kernel, config))
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", " ")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("%s_source_sha" % kernel) != kernel_sha(kernel):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# sources each measured kernel is built from (for matching counter summaries)
KERNEL_SOURCES = {
    "combine": ("combine.hip", "device.h", "launch.h"),
    "dispatch_fp8": ("dispatch.hip", "rows.h", "device.h", "launch.h"),
    "dispatch_bf16": ("dispatch.hip", "rows.h", "device.h", "launch.h"),
}


def kernel_sha(kernel: str) -> str:
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(root, "combine_group_limited_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def host_cpu():
    """CPU model and the threads this process may use (the machine's CPU share:
    the smaller of the affinity set and OMP_NUM_THREADS when it is set)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    use = min(avail, int(omp)) if omp.isdigit() and int(omp) > 0 else avail
    return {"cpu_model": model, "cpus_visible": os.cpu_count(), "cpus_affinity": avail, "threads": use}


def provenance(w, arrays):
    """Seeds and input hashes of the synthetic batch."""
    import numpy as np

    import workloads as W
    return {"seed": w.seed, "generator": "numpy %s PCG64, SeedSequence(seed).spawn(4): x, logits, y, bias"
            % np.__version__, "sha256": {k: W.sha256(v) for k, v in arrays.items()}}


def oracle_parity(w, fp8, gpu, lg, x, y):
    """The oracle's outputs on the bench's own batch against the GPU's
    (buffer set 0 after the timed steps): bit-exact for every integer output,
    the weights, payload and scales; combine counted in bf16 ulps.  Returns
    (parity record, the oracle's route and layout for the timing legs)."""
    import numpy as np

    import oracle

    def ordinal(b):  # bf16 patterns -> integers monotone in value, +0 and -0 both 0
        b = np.asarray(b, dtype=np.uint16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)

    idx, wt = oracle.route(lg, w.G, w.TG, w.k, w.topm)
    lay = oracle.layout(idx, w.E, w.R)
    checks = {"idx": (gpu["idx"], idx), "w": (gpu["wt"].view(np.uint32), wt.view(np.uint32)),
              "cnt": (gpu["cnt"], lay["cnt"]), "off": (gpu["off"], lay["off"]),
              "ntok_rank": (gpu["ntok"], lay["ntok_rank"]), "slot": (gpu["slot"], lay["slot"]),
              "recv_token": (gpu["recv_token"], lay["recv_token"])}
    if fp8:
        q, sc = oracle.dispatch_fp8(x, lay["slot"], w.nrows)
        checks["payload"] = (gpu["recv"], q)
        checks["scales"] = (gpu["scales"].view(np.uint32), sc.view(np.uint32))
    else:
        checks["payload"] = (gpu["recv"], oracle.dispatch_bf16(x, lay["slot"], w.nrows))
    rec = {}
    for k, (g, o) in checks.items():
        n = int(np.count_nonzero(np.asarray(g).ravel() != np.asarray(o).ravel()))
        rec[k] = "bit-exact" if n == 0 else "%d of %d differ" % (n, np.asarray(o).size)
    d = np.abs(ordinal(gpu["out"]) - ordinal(oracle.combine(y, lay["slot"], wt)))
    rec["combine_max_ulp"] = int(d.max()) if d.size else 0
    rec["combine_elements_differing"] = int((d > 0).sum())
    ok = all(v == "bit-exact" for k, v in rec.items() if not k.startswith("combine")) and rec["combine_max_ulp"] <= 1
    rec["verdict"] = "pass" if ok else "FAIL"
    rec["bar"] = "bit-exact routing, weights, layout, payload and scales; combine within 1 bf16 ulp"
    return rec, idx, wt, lay


def cpu_baseline(w, fp8, x, y, wt, lay, seconds: float):
    """The CPU oracle (plain single-threaded C, unchanged) timed on the same
    batch: dispatch + combine passes over the whole batch, on one thread and
    on every thread the host gives this process (the oracle's own functions
    called on token slices from a thread pool; ctypes releases the GIL).
    Each leg repeats passes for about half of `seconds`."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    q = np.empty((w.nrows, w.H), np.uint8 if fp8 else np.uint16)
    sc = np.empty((w.nrows, w.H // 128), np.float32)
    out = np.empty((w.T, w.H), np.uint16)
    slot = lay["slot"]
    nbytes = (w.bytes_dispatch_fp8() if fp8 else w.bytes_dispatch_bf16()) + w.bytes_combine()

    def part(t0, t1):
        if fp8:
            oracle.dispatch_fp8(x[t0:t1], slot[t0:t1], w.nrows, q, sc)
        else:
            oracle.dispatch_bf16(x[t0:t1], slot[t0:t1], w.nrows, q)
        out[t0:t1] = oracle.combine(y, slot[t0:t1], wt[t0:t1])

    def leg(threads):
        times = []
        t_start = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as pool:
            cuts = np.linspace(0, w.T, 4 * threads + 1).astype(int) if threads > 1 else np.array([0, w.T])
            while True:
                t0 = time.perf_counter()
                if threads == 1:
                    part(0, w.T)
                else:
                    list(pool.map(lambda i: part(cuts[i], cuts[i + 1]), range(len(cuts) - 1)))
                times.append(time.perf_counter() - t0)
                if time.perf_counter() - t_start >= seconds / 2 or len(times) >= 64:
                    break
        t = float(np.median(times))
        return round(nbytes / t / 1e9, 4), t, len(times)

    host = host_cpu()
    one, t1, n1 = leg(1)
    many, tn, nn = leg(host["threads"])
    kind = "FP8" if fp8 else "BF16"
    return {"value": many, "unit": "GB/s", "cores": host["threads"], "kind": "oracle",
            "sample": "full %s batch (%d tokens), %s dispatch + combine, median of %d passes of %.3f s on %d "
                      "threads (token slices)" % (w.name, w.T, kind, nn, tn, host["threads"]),
            "one_thread": {"value": one, "unit": "GB/s", "cores": 1,
                           "sample": "median of %d passes of %.3f s" % (n1, t1)},
            "host": host, "speedup_vs_one_thread": round(many / one, 2)}


if __name__ == "__main__":
    sys.exit(main())
