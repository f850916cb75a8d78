"""Python binding of the C ABI: ep_route, ep_get_layout, ep_dispatch,
ep_combine, with torch tensors for device memory and torch streams.

Argument marshalling only: shapes, dtypes, devices and contiguity are
checked here (the C ABI sees bare pointers and cannot), outputs are
allocated with torch.empty when not given, and every computation runs in
libep.so's kernels on the caller's current stream (or `stream`).

With an explicit `stream` that is not torch's current stream, the caller
keeps every tensor a call reads or returns alive until the work on that
stream has finished (for example until a synchronisation), as the C ABI
requires: torch's caching allocator only orders reuse of freed memory on
the current stream.  (Tensor.record_stream is no substitute for streams the
caller destroys, such as CuRangeStream: the allocator would later record
events on the destroyed stream.)  A layout call that allocates its own
workspace returns it in its dict under "workspace" for that reason: the
kernels on `stream` may still use it after the call returns.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib as L


class EpError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = L.lib().ep_strerror(code).decode()
        extra = ""
        if code == L.EP_ERR_HIP:
            extra = " (hipError %d)" % L.lib().ep_last_hip_error()
        super().__init__("%s: %s%s" % (where, msg, extra))
        self.code = code


@dataclasses.dataclass(frozen=True)
class Config:
    """Problem description (ep_config_t)."""
    T: int   # tokens
    H: int   # hidden size
    E: int   # experts
    G: int   # expert groups
    TG: int  # groups kept per token
    k: int   # experts per token
    R: int   # virtual expert ranks
    m: int = 0  # scores summed per group score (0 -> max(1, k // TG))

    def c(self) -> L.EpConfig:
        return L.EpConfig(self.T, self.H, self.E, self.G, self.TG, self.k, self.R, self.m)

    @property
    def nrows(self) -> int:
        return self.T * self.k

    @classmethod
    def of(cls, w) -> "Config":
        """From any object with T, H, E, G, TG, k, R, m attributes."""
        return cls(w.T, w.H, w.E, w.G, w.TG, w.k, w.R, w.m)


def _check(code: int, where: str) -> None:
    if code != L.EP_OK:
        raise EpError(code, where)


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _want(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError("%s must be on %s" % (name, device or "a GPU"))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def validate(cfg: Config) -> None:
    c = cfg.c()
    _check(L.lib().ep_validate_config(ctypes.byref(c)), "ep_validate_config")


def route(cfg: Config, logits: torch.Tensor, topk_idx=None, topk_w=None, stream=None):
    """Group-limited top-k gating. logits fp32 [T, E] -> (int32 [T, k], fp32 [T, k])."""
    dev = logits.device
    _want(logits, "logits", (cfg.T, cfg.E), torch.float32, None)
    if topk_idx is None:
        topk_idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    _want(topk_idx, "topk_idx", (cfg.T, cfg.k), torch.int32, dev)
    _want(topk_w, "topk_w", (cfg.T, cfg.k), torch.float32, dev)
    c = cfg.c()
    _check(L.lib().ep_route(ctypes.byref(c), _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                            _stream(stream, dev)), "ep_route")
    return topk_idx, topk_w


def scores(cfg: Config, logits: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """The gate's sigmoid scores, fp32 [T, E], bit-equal to those ep_route
    ranks.  `out` may be `logits` itself (in place)."""
    dev = logits.device
    _want(logits, "logits", (cfg.T, cfg.E), torch.float32, None)
    if out is None:
        out = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    _want(out, "scores", (cfg.T, cfg.E), torch.float32, dev)
    c = cfg.c()
    _check(L.lib().ep_scores(ctypes.byref(c), _ptr(logits), _ptr(out), _stream(stream, dev)), "ep_scores")
    return out


def layout_workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(L.lib().ep_layout_workspace_bytes(ctypes.byref(c)))


def get_layout(cfg: Config, topk_idx: torch.Tensor, out: dict | None = None, workspace=None,
               with_recv_token: bool = True, stream=None) -> dict:
    """Routing layout. Returns dict with cnt [E], ntok_rank [R], off [E+1],
    slot [T, k] and (if requested) recv_token [T*k], all int32, and the
    workspace when the call allocated it."""
    dev = topk_idx.device
    _want(topk_idx, "topk_idx", (cfg.T, cfg.k), torch.int32, None)
    o = dict(out or {})
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("cnt", torch.empty(cfg.E, **i32))
    o.setdefault("ntok_rank", torch.empty(cfg.R, **i32))
    o.setdefault("off", torch.empty(cfg.E + 1, **i32))
    o.setdefault("slot", torch.empty((cfg.T, cfg.k), **i32))
    if with_recv_token:
        o.setdefault("recv_token", torch.empty(cfg.T * cfg.k, **i32))
    _want(o["cnt"], "cnt", (cfg.E,), torch.int32, dev)
    _want(o["ntok_rank"], "ntok_rank", (cfg.R,), torch.int32, dev)
    _want(o["off"], "off", (cfg.E + 1,), torch.int32, dev)
    _want(o["slot"], "slot", (cfg.T, cfg.k), torch.int32, dev)
    rt = o.get("recv_token")
    if rt is not None:
        _want(rt, "recv_token", (cfg.T * cfg.k,), torch.int32, dev)
    need = layout_workspace_bytes(cfg)
    if workspace is None:
        workspace = o["workspace"] = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    c = cfg.c()
    _check(L.lib().ep_get_layout(ctypes.byref(c), _ptr(topk_idx), _ptr(o["cnt"]), _ptr(o["ntok_rank"]),
                                 _ptr(o["off"]), _ptr(o["slot"]), _ptr(rt), _ptr(workspace),
                                 workspace.numel(), _stream(stream, dev)), "ep_get_layout")
    return o


def route_layout_workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(L.lib().ep_route_layout_workspace_bytes(ctypes.byref(c)))


def route_layout(cfg: Config, logits: torch.Tensor, out: dict | None = None, workspace=None,
                 with_recv_token: bool = True, stream=None) -> dict:
    """route followed by get_layout, in fewer launches, with the same
    results: a dict with idx [T, k] int32, w [T, k] fp32 and the layout's
    cnt, ntok_rank, off, slot and (if requested) recv_token, and the
    workspace when the call allocated it."""
    dev = logits.device
    _want(logits, "logits", (cfg.T, cfg.E), torch.float32, None)
    o = dict(out or {})
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("idx", torch.empty((cfg.T, cfg.k), **i32))
    o.setdefault("w", torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev))
    o.setdefault("cnt", torch.empty(cfg.E, **i32))
    o.setdefault("ntok_rank", torch.empty(cfg.R, **i32))
    o.setdefault("off", torch.empty(cfg.E + 1, **i32))
    o.setdefault("slot", torch.empty((cfg.T, cfg.k), **i32))
    if with_recv_token:
        o.setdefault("recv_token", torch.empty(cfg.T * cfg.k, **i32))
    _want(o["idx"], "idx", (cfg.T, cfg.k), torch.int32, dev)
    _want(o["w"], "w", (cfg.T, cfg.k), torch.float32, dev)
    _want(o["cnt"], "cnt", (cfg.E,), torch.int32, dev)
    _want(o["ntok_rank"], "ntok_rank", (cfg.R,), torch.int32, dev)
    _want(o["off"], "off", (cfg.E + 1,), torch.int32, dev)
    _want(o["slot"], "slot", (cfg.T, cfg.k), torch.int32, dev)
    rt = o.get("recv_token")
    if rt is not None:
        _want(rt, "recv_token", (cfg.T * cfg.k,), torch.int32, dev)
    need = route_layout_workspace_bytes(cfg)
    if workspace is None:
        workspace = o["workspace"] = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    c = cfg.c()
    _check(L.lib().ep_route_layout(ctypes.byref(c), _ptr(logits), _ptr(o["idx"]), _ptr(o["w"]), _ptr(o["cnt"]),
                                   _ptr(o["ntok_rank"]), _ptr(o["off"]), _ptr(o["slot"]), _ptr(rt),
                                   _ptr(workspace), workspace.numel(), _stream(stream, dev)), "ep_route_layout")
    return o


def get_layout_static(cfg: Config, topk_idx: torch.Tensor, out: dict | None = None,
                      with_recv_token: bool = True, stream=None) -> dict:
    """get_layout without a workspace: the library's static device scratch
    (at most EP_STATIC_SCRATCH_BYTES) stands in for it, so the call
    allocates nothing when `out` holds every output.  Calls that may overlap
    on one GPU race on that scratch."""
    dev = topk_idx.device
    _want(topk_idx, "topk_idx", (cfg.T, cfg.k), torch.int32, None)
    o = dict(out or {})
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("cnt", torch.empty(cfg.E, **i32))
    o.setdefault("ntok_rank", torch.empty(cfg.R, **i32))
    o.setdefault("off", torch.empty(cfg.E + 1, **i32))
    o.setdefault("slot", torch.empty((cfg.T, cfg.k), **i32))
    if with_recv_token:
        o.setdefault("recv_token", torch.empty(cfg.T * cfg.k, **i32))
    _want(o["cnt"], "cnt", (cfg.E,), torch.int32, dev)
    _want(o["ntok_rank"], "ntok_rank", (cfg.R,), torch.int32, dev)
    _want(o["off"], "off", (cfg.E + 1,), torch.int32, dev)
    _want(o["slot"], "slot", (cfg.T, cfg.k), torch.int32, dev)
    rt = o.get("recv_token")
    if rt is not None:
        _want(rt, "recv_token", (cfg.T * cfg.k,), torch.int32, dev)
    c = cfg.c()
    _check(L.lib().ep_get_layout_static(ctypes.byref(c), _ptr(topk_idx), _ptr(o["cnt"]), _ptr(o["ntok_rank"]),
                                        _ptr(o["off"]), _ptr(o["slot"]), _ptr(rt), _stream(stream, dev)),
           "ep_get_layout_static")
    return o


def dispatch(cfg: Config, x: torch.Tensor, slot: torch.Tensor, recv_dtype: str = "fp8", recv=None,
             recv_scales=None, stream=None):
    """Dispatch bf16 x [T, H] to T*k receive rows.  fp8: returns (recv uint8
    [T*k, H] of E4M3 codes, scales fp32 [T*k, H/128]); bf16: returns (recv
    bf16 [T*k, H], None).  Rows no slot names are left as they were."""
    dev = x.device
    _want(x, "x", (cfg.T, cfg.H), torch.bfloat16, None)
    _want(slot, "slot", (cfg.T, cfg.k), torch.int32, dev)
    if recv_dtype == "fp8":
        if recv is None:
            recv = torch.empty((cfg.nrows, cfg.H), dtype=torch.uint8, device=dev)
        if recv_scales is None:
            recv_scales = torch.empty((cfg.nrows, cfg.H // 128), dtype=torch.float32, device=dev)
        if recv.dtype == torch.float8_e4m3fn:
            recv_u8 = recv.view(torch.uint8)
        else:
            recv_u8 = recv
        _want(recv_u8, "recv", (cfg.nrows, cfg.H), torch.uint8, dev)
        _want(recv_scales, "recv_scales", (cfg.nrows, cfg.H // 128), torch.float32, dev)
        code = L.EP_RECV_FP8_E4M3
    elif recv_dtype == "bf16":
        if recv is None:
            recv = torch.empty((cfg.nrows, cfg.H), dtype=torch.bfloat16, device=dev)
        _want(recv, "recv", (cfg.nrows, cfg.H), torch.bfloat16, dev)
        if recv_scales is not None:
            raise ValueError("recv_scales must be None for bf16 dispatch")
        code = L.EP_RECV_BF16
    else:
        raise ValueError("recv_dtype must be 'fp8' or 'bf16'")
    c = cfg.c()
    _check(L.lib().ep_dispatch(ctypes.byref(c), _ptr(x), _ptr(slot), code, _ptr(recv), _ptr(recv_scales),
                               _stream(stream, dev)), "ep_dispatch")
    return recv, recv_scales


def combine(cfg: Config, y: torch.Tensor, slot: torch.Tensor, topk_w: torch.Tensor, out=None, stream=None):
    """Weighted combine of bf16 expert outputs y [T*k, H] -> bf16 [T, H]."""
    dev = y.device
    _want(y, "y", (cfg.nrows, cfg.H), torch.bfloat16, None)
    _want(slot, "slot", (cfg.T, cfg.k), torch.int32, dev)
    _want(topk_w, "topk_w", (cfg.T, cfg.k), torch.float32, dev)
    if out is None:
        out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    _want(out, "out", (cfg.T, cfg.H), torch.bfloat16, dev)
    c = cfg.c()
    _check(L.lib().ep_combine(ctypes.byref(c), _ptr(y), _ptr(slot), _ptr(topk_w), _ptr(out),
                              _stream(stream, dev)), "ep_combine")
    return out


def dispatch_ll(cfg: Config, x: torch.Tensor, topk_idx: torch.Tensor, capacity: int, recv_dtype: str = "fp8",
                recv=None, recv_scales=None, recv_count=None, recv_src=None, slot=None, stream=None) -> dict:
    """Low-latency dispatch into fixed-capacity per-expert receive rows
    (expert e owns rows [e*capacity, (e+1)*capacity)).  Returns a dict with
    recv ([E*capacity, H] uint8 E4M3 codes or bf16), scales (fp32
    [E*capacity, H/128] or None), count (int32 [E]), src (int32
    [E*capacity]) and slot (int32 [T, k]).  Rows no pair takes, and their
    src entries, are left as they were."""
    dev = x.device
    _want(x, "x", (cfg.T, cfg.H), torch.bfloat16, None)
    _want(topk_idx, "topk_idx", (cfg.T, cfg.k), torch.int32, dev)
    nrows = cfg.E * capacity
    i32 = dict(dtype=torch.int32, device=dev)
    if recv_dtype == "fp8":
        if recv is None:
            recv = torch.empty((nrows, cfg.H), dtype=torch.uint8, device=dev)
        if recv_scales is None:
            recv_scales = torch.empty((nrows, cfg.H // 128), dtype=torch.float32, device=dev)
        recv_u8 = recv.view(torch.uint8) if recv.dtype == torch.float8_e4m3fn else recv
        _want(recv_u8, "recv", (nrows, cfg.H), torch.uint8, dev)
        _want(recv_scales, "recv_scales", (nrows, cfg.H // 128), torch.float32, dev)
        code = L.EP_RECV_FP8_E4M3
    elif recv_dtype == "bf16":
        if recv is None:
            recv = torch.empty((nrows, cfg.H), dtype=torch.bfloat16, device=dev)
        _want(recv, "recv", (nrows, cfg.H), torch.bfloat16, dev)
        if recv_scales is not None:
            raise ValueError("recv_scales must be None for bf16 dispatch")
        code = L.EP_RECV_BF16
    else:
        raise ValueError("recv_dtype must be 'fp8' or 'bf16'")
    if recv_count is None:
        recv_count = torch.empty(cfg.E, **i32)
    if recv_src is None:
        recv_src = torch.empty(nrows, **i32)
    if slot is None:
        slot = torch.empty((cfg.T, cfg.k), **i32)
    _want(recv_count, "recv_count", (cfg.E,), torch.int32, dev)
    _want(recv_src, "recv_src", (nrows,), torch.int32, dev)
    _want(slot, "slot", (cfg.T, cfg.k), torch.int32, dev)
    c = cfg.c()
    _check(L.lib().ep_dispatch_ll(ctypes.byref(c), _ptr(x), _ptr(topk_idx), capacity, code, _ptr(recv),
                                  _ptr(recv_scales), _ptr(recv_count), _ptr(recv_src), _ptr(slot),
                                  _stream(stream, dev)), "ep_dispatch_ll")
    return dict(recv=recv, scales=recv_scales, count=recv_count, src=recv_src, slot=slot)


def combine_ll(cfg: Config, capacity: int, y: torch.Tensor, slot: torch.Tensor, topk_w: torch.Tensor, out=None,
               stream=None):
    """Weighted combine of bf16 expert outputs in ep_dispatch_ll's receive
    rows, y [E*capacity, H] -> bf16 [T, H]."""
    dev = y.device
    _want(y, "y", (cfg.E * capacity, cfg.H), torch.bfloat16, None)
    _want(slot, "slot", (cfg.T, cfg.k), torch.int32, dev)
    _want(topk_w, "topk_w", (cfg.T, cfg.k), torch.float32, dev)
    if out is None:
        out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    _want(out, "out", (cfg.T, cfg.H), torch.bfloat16, dev)
    c = cfg.c()
    _check(L.lib().ep_combine_ll(ctypes.byref(c), capacity, _ptr(y), _ptr(slot), _ptr(topk_w), _ptr(out),
                                 _stream(stream, dev)), "ep_combine_ll")
    return out


def rank_layout_workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(L.lib().ep_rank_layout_workspace_bytes(ctypes.byref(c)))


def get_rank_layout(cfg: Config, topk_idx: torch.Tensor, out: dict | None = None, workspace=None,
                    with_rank_token: bool = True, stream=None) -> dict:
    """Per-rank deduplicated layout: dict with rank_count [R], rank_offset
    [R+1], rank_slot [T, k] and (if requested) rank_token [T*k], all int32,
    and the workspace when the call allocated it.  ep_dispatch with
    rank_slot as the slot map is the deduplicated dispatch."""
    dev = topk_idx.device
    _want(topk_idx, "topk_idx", (cfg.T, cfg.k), torch.int32, None)
    o = dict(out or {})
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("rank_count", torch.empty(cfg.R, **i32))
    o.setdefault("rank_offset", torch.empty(cfg.R + 1, **i32))
    o.setdefault("rank_slot", torch.empty((cfg.T, cfg.k), **i32))
    if with_rank_token:
        o.setdefault("rank_token", torch.empty(cfg.T * cfg.k, **i32))
    _want(o["rank_count"], "rank_count", (cfg.R,), torch.int32, dev)
    _want(o["rank_offset"], "rank_offset", (cfg.R + 1,), torch.int32, dev)
    _want(o["rank_slot"], "rank_slot", (cfg.T, cfg.k), torch.int32, dev)
    rt = o.get("rank_token")
    if rt is not None:
        _want(rt, "rank_token", (cfg.T * cfg.k,), torch.int32, dev)
    need = rank_layout_workspace_bytes(cfg)
    if workspace is None:
        workspace = o["workspace"] = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    c = cfg.c()
    _check(L.lib().ep_get_rank_layout(ctypes.byref(c), _ptr(topk_idx), _ptr(o["rank_count"]), _ptr(o["rank_offset"]),
                                      _ptr(o["rank_slot"]), _ptr(rt), _ptr(workspace), workspace.numel(),
                                      _stream(stream, dev)), "ep_get_rank_layout")
    return o


def combine_rank_partial(cfg: Config, y: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
                         topk_w: torch.Tensor, rank_slot: torch.Tensor, partial=None, stream=None):
    """In-rank partial combine: bf16 partial rows [T*k, H] (rows no
    rank_slot names are left as they were)."""
    dev = y.device
    _want(y, "y", (cfg.nrows, cfg.H), torch.bfloat16, None)
    for name, t in (("topk_idx", topk_idx), ("slot", slot), ("rank_slot", rank_slot)):
        _want(t, name, (cfg.T, cfg.k), torch.int32, dev)
    _want(topk_w, "topk_w", (cfg.T, cfg.k), torch.float32, dev)
    if partial is None:
        partial = torch.empty((cfg.nrows, cfg.H), dtype=torch.bfloat16, device=dev)
    _want(partial, "partial", (cfg.nrows, cfg.H), torch.bfloat16, dev)
    c = cfg.c()
    _check(L.lib().ep_combine_rank_partial(ctypes.byref(c), _ptr(y), _ptr(topk_idx), _ptr(slot), _ptr(topk_w),
                                           _ptr(rank_slot), _ptr(partial), _stream(stream, dev)),
           "ep_combine_rank_partial")
    return partial


def combine_ranks(cfg: Config, partial: torch.Tensor, rank_slot: torch.Tensor, out=None, stream=None):
    """Sum of each token's partial rows -> bf16 [T, H]."""
    dev = partial.device
    _want(partial, "partial", (cfg.nrows, cfg.H), torch.bfloat16, None)
    _want(rank_slot, "rank_slot", (cfg.T, cfg.k), torch.int32, dev)
    if out is None:
        out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    _want(out, "out", (cfg.T, cfg.H), torch.bfloat16, dev)
    c = cfg.c()
    _check(L.lib().ep_combine_ranks(ctypes.byref(c), _ptr(partial), _ptr(rank_slot), _ptr(out),
                                    _stream(stream, dev)), "ep_combine_ranks")
    return out


class CuRangeStream:
    """A HIP stream confined to compute units [first_cu, first_cu + num_cus)
    (ep_stream_create_cu_range), usable as `stream=` here and, through
    `.torch`, as a torch stream.  Release it with close() (or a with-block)
    after its work has been waited for."""

    def __init__(self, first_cu: int, num_cus: int):
        h = ctypes.c_void_p()
        _check(L.lib().ep_stream_create_cu_range(first_cu, num_cus, ctypes.byref(h)), "ep_stream_create_cu_range")
        self.handle = h.value
        self.first_cu, self.num_cus = first_cu, num_cus
        self.torch = torch.cuda.ExternalStream(self.handle)

    @property
    def cuda_stream(self) -> int:
        return self.handle

    def close(self) -> None:
        if self.handle:
            _check(L.lib().ep_stream_destroy(self.handle), "ep_stream_destroy")
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        torch.cuda.synchronize()
        self.close()
