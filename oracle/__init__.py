"""Plain CPU oracle for MoE routing, layout, dispatch and combine.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product library
never does, and it shares no code with it.  The arithmetic lives in
``oracle.c`` (plain single-threaded C, fp32 exactly as written, no implicit
fused multiply-add); this module only builds it with gcc and marshals numpy
arrays through ctypes.

Every function mirrors one C entry point; the C file states the reading of
the DeepEP pages each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc)."""
    stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I = ctypes.c_int
        F = ctypes.c_float
        L.orc_expf.argtypes = [F]; L.orc_expf.restype = F
        L.orc_sigmoid.argtypes = [F]; L.orc_sigmoid.restype = F
        L.orc_expf_hi.argtypes = []; L.orc_expf_hi.restype = F
        L.orc_expf_lo.argtypes = []; L.orc_expf_lo.restype = F
        L.orc_e4m3_from_f32.argtypes = [F]; L.orc_e4m3_from_f32.restype = ctypes.c_uint8
        L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]; L.orc_e4m3_to_f32.restype = F
        L.orc_bf16_from_f32.argtypes = [F]; L.orc_bf16_from_f32.restype = ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]; L.orc_bf16_to_f32.restype = F
        L.orc_expf_n.argtypes = [ctypes.c_long, P, P]; L.orc_expf_n.restype = None
        L.orc_e4m3_from_f32_n.argtypes = [ctypes.c_long, P, P]; L.orc_e4m3_from_f32_n.restype = None
        L.orc_bf16_from_f32_n.argtypes = [ctypes.c_long, P, P]; L.orc_bf16_from_f32_n.restype = None
        L.orc_scores.argtypes = [I, I, P, P]; L.orc_scores.restype = None
        L.orc_select.argtypes = [I, I, I, I, I, I, P, P, P]; L.orc_select.restype = I
        L.orc_route.argtypes = [I, I, I, I, I, I, P, P, P]; L.orc_route.restype = I
        L.orc_layout.argtypes = [I, I, I, I, P, P, P, P, P, P]; L.orc_layout.restype = I
        L.orc_ll_layout.argtypes = [I, I, I, I, P, P, P, P]; L.orc_ll_layout.restype = I
        L.orc_rank_layout.argtypes = [I, I, I, I, P, P, P, P, P]; L.orc_rank_layout.restype = I
        L.orc_combine_rank_partial.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, P]
        L.orc_combine_rank_partial.restype = None
        L.orc_combine_ranks.argtypes = [I, I, I, I, P, P, P]; L.orc_combine_ranks.restype = None
        L.orc_dispatch_fp8.argtypes = [I, I, I, I, P, P, P, P]; L.orc_dispatch_fp8.restype = None
        L.orc_dispatch_bf16.argtypes = [I, I, I, I, P, P, P]; L.orc_dispatch_bf16.restype = None
        L.orc_combine.argtypes = [I, I, I, I, P, P, P, P]; L.orc_combine.restype = None
        L.orc_combine_f64.argtypes = [I, I, I, I, P, P, P, P]; L.orc_combine_f64.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar helpers, vectorised by a plain loop ---------------------------

def expf(x) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.float32)
    lib().orc_expf_n(x.size, _p(x), _p(y))
    return y


def sigmoid(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.float32)
    if x.size:
        lib().orc_scores(1, x.size, _p(x), _p(out))
    return out


def e4m3_from_f32(v) -> np.ndarray:
    v = _c(v, np.float32)
    c = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_from_f32_n(v.size, _p(v), _p(c))
    return c


def e4m3_to_f32(c) -> np.ndarray:
    c = _c(c, np.uint8).ravel()
    f = lib().orc_e4m3_to_f32
    return np.array([f(int(a)) for a in c], dtype=np.float32)


def bf16_from_f32(v) -> np.ndarray:
    v = _c(v, np.float32)
    b = np.empty(v.shape, np.uint16)
    lib().orc_bf16_from_f32_n(v.size, _p(v), _p(b))
    return b


def bf16_to_f32(b) -> np.ndarray:
    b = _c(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---- the four steps --------------------------------------------------------

def scores(logits) -> np.ndarray:
    logits = _c(logits, np.float32)
    T, E = logits.shape
    s = np.empty((T, E), np.float32)
    lib().orc_scores(T, E, _p(logits), _p(s))
    return s


def select(s, G: int, TG: int, k: int, m: int = 0):
    s = _c(s, np.float32)
    T, E = s.shape
    m = m or k // TG
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = lib().orc_select(T, E, G, TG, k, m, _p(s), _p(idx), _p(w))
    if rc != 0:
        raise ValueError("invalid gating configuration")
    return idx, w


def route(logits, G: int, TG: int, k: int, m: int = 0):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    m = m or k // TG
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = lib().orc_route(T, E, G, TG, k, m, _p(logits), _p(idx), _p(w))
    if rc != 0:
        raise ValueError("invalid gating configuration")
    return idx, w


def layout(topk_idx, E: int, R: int):
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    cnt = np.empty(E, np.int32)
    off = np.empty(E + 1, np.int32)
    ntok = np.empty(R, np.int32)
    slot = np.empty((T, k), np.int32)
    recv_token = np.empty(T * k, np.int32)
    rc = lib().orc_layout(T, k, E, R, _p(idx), _p(cnt), _p(off), _p(ntok), _p(slot), _p(recv_token))
    if rc != 0:
        raise ValueError("invalid layout configuration")
    return dict(cnt=cnt, off=off, ntok_rank=ntok, slot=slot, recv_token=recv_token)


def ll_layout(topk_idx, E: int, cap: int, src=None):
    """Low-latency layout: returns dict(count [E], slot [T, k], src [E*cap]);
    src entries of rows no pair takes keep the given array's values (-1 if
    none is given)."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    count = np.empty(E, np.int32)
    slot = np.empty((T, k), np.int32)
    if src is None:
        src = np.full(E * cap, -1, np.int32)
    src = _c(src, np.int32)
    rc = lib().orc_ll_layout(T, k, E, cap, _p(idx), _p(count), _p(slot), _p(src))
    if rc != 0:
        raise ValueError("invalid low-latency layout configuration")
    return dict(count=count, slot=slot, src=src)


def dispatch_fp8(x_bf16, slot, nrows: int, q=None, sc=None):
    """x_bf16: uint16 [T, H]; returns (q uint8 [nrows, H], sc f32 [nrows, H/128]).
    Rows no slot names keep the contents of q / sc if given, else zero."""
    x = _c(x_bf16, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    k = slot.shape[1] if slot.ndim == 2 else 0
    if q is None:
        q = np.zeros((nrows, H), np.uint8)
    if sc is None:
        sc = np.zeros((nrows, H // 128), np.float32)
    lib().orc_dispatch_fp8(T, H, k, nrows, _p(x), _p(slot), _p(q), _p(sc))
    return q, sc


def dispatch_bf16(x_bf16, slot, nrows: int, recv=None):
    x = _c(x_bf16, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    k = slot.shape[1] if slot.ndim == 2 else 0
    if recv is None:
        recv = np.zeros((nrows, H), np.uint16)
    lib().orc_dispatch_bf16(T, H, k, nrows, _p(x), _p(slot), _p(recv))
    return recv


def combine(y_bf16, slot, w) -> np.ndarray:
    y = _c(y_bf16, np.uint16)
    slot = _c(slot, np.int32)
    w = _c(w, np.float32)
    nrows, H = y.shape
    T, k = slot.shape
    out = np.empty((T, H), np.uint16)
    lib().orc_combine(T, H, k, nrows, _p(y), _p(slot), _p(w), _p(out))
    return out


def combine_f64(y_bf16, slot, w) -> np.ndarray:
    y = _c(y_bf16, np.uint16)
    slot = _c(slot, np.int32)
    w = _c(w, np.float32)
    nrows, H = y.shape
    T, k = slot.shape
    out = np.empty((T, H), np.float64)
    lib().orc_combine_f64(T, H, k, nrows, _p(y), _p(slot), _p(w), _p(out))
    return out


def rank_layout(topk_idx, E: int, R: int):
    """Per-rank deduplicated layout: dict(rank_count [R], rank_offset [R+1],
    rank_slot [T, k], rank_token [T*k])."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    cnt = np.empty(R, np.int32)
    off = np.empty(R + 1, np.int32)
    rslot = np.empty((T, k), np.int32)
    rtok = np.empty(T * k, np.int32)
    rc = lib().orc_rank_layout(T, k, E, R, _p(idx), _p(cnt), _p(off), _p(rslot), _p(rtok))
    if rc != 0:
        raise ValueError("invalid rank layout configuration")
    return dict(rank_count=cnt, rank_offset=off, rank_slot=rslot, rank_token=rtok)


def combine_rank_partial(y_bf16, topk_idx, slot, w, rank_slot, E: int, R: int, nrows_partial: int, partial=None):
    """In-rank partial combine: uint16 partial rows [nrows_partial, H]; rows
    no rank_slot names keep `partial`'s values (zero if not given)."""
    y = _c(y_bf16, np.uint16)
    idx = _c(topk_idx, np.int32)
    slot = _c(slot, np.int32)
    w = _c(w, np.float32)
    rslot = _c(rank_slot, np.int32)
    nrows, H = y.shape
    T, k = idx.shape
    if partial is None:
        partial = np.zeros((nrows_partial, H), np.uint16)
    partial = _c(partial, np.uint16)
    lib().orc_combine_rank_partial(T, H, k, E, R, nrows, _p(y), _p(idx), _p(slot), _p(w), _p(rslot),
                                   nrows_partial, _p(partial))
    return partial


def combine_ranks(partial_bf16, rank_slot) -> np.ndarray:
    """Sum of each token's partial rows (first-pick order), rounded to bf16."""
    p = _c(partial_bf16, np.uint16)
    rslot = _c(rank_slot, np.int32)
    nrows_partial, H = p.shape
    T, k = rslot.shape
    out = np.empty((T, H), np.uint16)
    lib().orc_combine_ranks(T, H, k, nrows_partial, _p(p), _p(rslot), _p(out))
    return out
