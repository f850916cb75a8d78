"""C ABI checks that need no GPU: the library loads, exports every function
include/ep.h declares, and rejects invalid calls with the documented codes
before making any HIP call (so fake device addresses are safe here)."""
import ctypes
import os
import re

import pytest

import combine_group_limited_amd as ep
import workloads as W
from combine_group_limited_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ep.h")).read()
    return re.findall(r"EP_API\s+[\w\s\*]+?\b(ep_\w+)\s*\(", src)


def test_every_declared_function_is_exported():
    names = _declared()
    assert set(names) == set(L.EXPORTS), names
    lib = ep.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_version_and_messages():
    lib = ep.lib()
    assert lib.ep_abi_version() == 4
    for code in (0, -1, -2, -3, -4, -5, -6, 42):
        assert len(lib.ep_strerror(code)) > 0
    assert lib.ep_last_hip_error() == 0


def _cfg(**kw):
    base = dict(T=4096, H=7168, E=256, G=8, TG=4, k=8, R=32, m=0)
    base.update(kw)
    return ep.Config(**base)


@pytest.mark.parametrize("name", sorted(W.CONFIGS))
def test_workload_configs_are_valid(name):
    ep.validate(ep.Config.of(W.CONFIGS[name]))


@pytest.mark.parametrize("kw,code", [
    (dict(H=100), L.EP_ERR_INVALID_ARG),
    (dict(H=0), L.EP_ERR_INVALID_ARG),
    (dict(T=-1), L.EP_ERR_INVALID_ARG),
    (dict(E=250), L.EP_ERR_INVALID_ARG),          # not divisible by G
    (dict(TG=9), L.EP_ERR_INVALID_ARG),
    (dict(TG=0), L.EP_ERR_INVALID_ARG),
    (dict(k=0), L.EP_ERR_INVALID_ARG),
    (dict(TG=1, k=33), L.EP_ERR_INVALID_ARG),     # more than one group holds
    (dict(R=3), L.EP_ERR_INVALID_ARG),
    (dict(m=33), L.EP_ERR_INVALID_ARG),           # more than a group holds
    (dict(m=-1), L.EP_ERR_INVALID_ARG),
    (dict(T=1 << 28), L.EP_ERR_INVALID_ARG),      # T * k >= 2^31
    (dict(H=16384 + 128), L.EP_ERR_UNSUPPORTED),
    (dict(E=2048, G=64, R=32), L.EP_ERR_UNSUPPORTED),
    (dict(k=40, TG=8), L.EP_ERR_UNSUPPORTED),
    (dict(m=9, k=8, TG=1), L.EP_ERR_UNSUPPORTED),
    (dict(T=(1 << 24) + 1, k=1), L.EP_ERR_UNSUPPORTED),
])
def test_invalid_configs(kw, code):
    c = _cfg(**kw).c()
    assert ep.lib().ep_validate_config(ctypes.byref(c)) == code


def test_null_config():
    lib = ep.lib()
    assert lib.ep_validate_config(None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_route(None, 0x1000, 0x1000, 0x1000, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_layout_workspace_bytes(None) == 0


def test_workspace_size():
    a = ep.layout_workspace_bytes(_cfg(T=128))
    b = ep.layout_workspace_bytes(_cfg(T=4096))
    assert a > 0 and b > a and b % 256 == 0
    assert ep.layout_workspace_bytes(_cfg(H=100)) == 0


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation


def test_route_rejections():
    lib = ep.lib()
    c = _cfg().c()
    assert lib.ep_route(ctypes.byref(c), None, FAKE, FAKE, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_route(ctypes.byref(c), FAKE + 2, FAKE, FAKE, None) == L.EP_ERR_ALIGNMENT
    bad = _cfg(H=100).c()
    assert lib.ep_route(ctypes.byref(bad), FAKE, FAKE, FAKE, None) == L.EP_ERR_INVALID_ARG
    # nothing to do for zero tokens: succeeds without touching the GPU
    z = _cfg(T=0).c()
    assert lib.ep_route(ctypes.byref(z), None, None, None, None) == L.EP_OK


def test_scores_rejections():
    lib = ep.lib()
    c = _cfg().c()
    assert lib.ep_scores(ctypes.byref(c), None, FAKE, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_scores(ctypes.byref(c), FAKE, None, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_scores(ctypes.byref(c), FAKE + 2, FAKE, None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_scores(ctypes.byref(c), FAKE, FAKE + 1, None) == L.EP_ERR_ALIGNMENT
    bad = _cfg(H=100).c()
    assert lib.ep_scores(ctypes.byref(bad), FAKE, FAKE, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_scores(None, FAKE, FAKE, None) == L.EP_ERR_INVALID_ARG
    z = _cfg(T=0).c()
    assert lib.ep_scores(ctypes.byref(z), None, None, None) == L.EP_OK


def test_layout_rejections():
    lib = ep.lib()
    c = _cfg().c()
    need = lib.ep_layout_workspace_bytes(ctypes.byref(c))
    args = [FAKE] * 6
    assert lib.ep_get_layout(ctypes.byref(c), *args, FAKE, need - 1, None) == L.EP_ERR_WORKSPACE
    assert lib.ep_get_layout(ctypes.byref(c), *args, None, need, None) == L.EP_ERR_WORKSPACE
    assert lib.ep_get_layout(ctypes.byref(c), *args, FAKE + 4, need, None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_get_layout(ctypes.byref(c), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                             None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_get_layout(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE + 1, FAKE, FAKE, need,
                             None) == L.EP_ERR_ALIGNMENT


def test_route_layout_rejections():
    lib = ep.lib()
    c = _cfg().c()
    need = lib.ep_route_layout_workspace_bytes(ctypes.byref(c))
    assert need > 0
    # the two-launch path's workspace at prefill: a byte per expert and per
    # rank for each 16-token column
    assert need == 256 * 256 + 256 * 32
    args = [FAKE] * 8
    assert lib.ep_route_layout(ctypes.byref(c), *args, FAKE, need - 1, None) == L.EP_ERR_WORKSPACE
    assert lib.ep_route_layout(ctypes.byref(c), *args, None, need, None) == L.EP_ERR_WORKSPACE
    assert lib.ep_route_layout(ctypes.byref(c), *args, FAKE + 8, need, None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_route_layout(ctypes.byref(c), FAKE + 2, *args[1:], FAKE, need, None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_route_layout(ctypes.byref(c), None, *args[1:], FAKE, need, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_route_layout(ctypes.byref(c), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                               None) == L.EP_ERR_INVALID_ARG
    bad = _cfg(E=100).c()
    assert lib.ep_route_layout_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.ep_route_layout(ctypes.byref(bad), *args, FAKE, need, None) == L.EP_ERR_INVALID_ARG
    # other shapes need the layout's own workspace
    small = _cfg(T=64).c()
    assert lib.ep_route_layout_workspace_bytes(ctypes.byref(small)) == lib.ep_layout_workspace_bytes(ctypes.byref(small))


def test_layout_static_rejections():
    # validated before any HIP call, so fake device addresses are safe here
    lib = ep.lib()
    c = _cfg().c()
    assert lib.ep_layout_workspace_bytes(ctypes.byref(c)) <= L.EP_STATIC_SCRATCH_BYTES
    args = [FAKE] * 6
    assert lib.ep_get_layout_static(None, *args, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_get_layout_static(ctypes.byref(c), FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                    None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_get_layout_static(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE,
                                    None) == L.EP_ERR_ALIGNMENT
    # beyond the static scratch: the largest T whose workspace fits passes
    # validation of the size, one more count block does not
    E, R, k = 256, 32, 8
    fits = (L.EP_STATIC_SCRATCH_BYTES // (4 * (E + R))) * 512 // k
    big = _cfg(T=fits + 512 // k).c()
    assert lib.ep_layout_workspace_bytes(ctypes.byref(big)) > L.EP_STATIC_SCRATCH_BYTES
    assert lib.ep_get_layout_static(ctypes.byref(big), *args, None) == L.EP_ERR_SCRATCH_LIMIT
    msg = lib.ep_strerror(L.EP_ERR_SCRATCH_LIMIT).decode()
    assert "ep_get_layout" in msg and "scratch" in msg
    ok = _cfg(T=fits).c()
    assert lib.ep_layout_workspace_bytes(ctypes.byref(ok)) <= L.EP_STATIC_SCRATCH_BYTES


def test_dispatch_rejections():
    lib = ep.lib()
    c = _cfg().c()
    assert lib.ep_dispatch(ctypes.byref(c), FAKE, FAKE, 7, FAKE, FAKE, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(c), FAKE, FAKE, L.EP_RECV_FP8_E4M3, FAKE, None,
                           None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(c), FAKE, FAKE, L.EP_RECV_BF16, FAKE, FAKE,
                           None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(c), FAKE + 8, FAKE, L.EP_RECV_FP8_E4M3, FAKE, FAKE,
                           None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_dispatch(ctypes.byref(c), FAKE, FAKE, L.EP_RECV_BF16, FAKE + 4, None,
                           None) == L.EP_ERR_ALIGNMENT


def test_combine_rejections():
    lib = ep.lib()
    c = _cfg().c()
    assert lib.ep_combine(ctypes.byref(c), FAKE, FAKE, FAKE, None, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_combine(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE + 8, None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_combine(ctypes.byref(c), FAKE, FAKE + 2, FAKE, FAKE, None) == L.EP_ERR_ALIGNMENT
    z = _cfg(T=0).c()
    assert lib.ep_combine(ctypes.byref(z), None, None, None, None, None) == L.EP_OK


def test_low_latency_rejections():
    lib = ep.lib()
    c = _cfg(T=128).c()
    F8, B16 = L.EP_RECV_FP8_E4M3, L.EP_RECV_BF16
    ok = [FAKE, FAKE, 128, F8, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    def call(cfg, *over):
        a = list(ok)
        for i, v in over:
            a[i] = v
        return lib.ep_dispatch_ll(ctypes.byref(cfg), *a)
    assert call(c, (2, 0)) == L.EP_ERR_INVALID_ARG                    # capacity 0
    assert call(c, (2, 1 << 23)) == L.EP_ERR_INVALID_ARG              # E * capacity >= 2^31
    assert call(c, (3, 5)) == L.EP_ERR_INVALID_ARG                    # unknown payload type
    assert call(c, (6, None)) == L.EP_ERR_INVALID_ARG                 # no recv_count
    assert call(c, (5, None)) == L.EP_ERR_INVALID_ARG                 # FP8 without scales
    assert call(c, (3, B16)) == L.EP_ERR_INVALID_ARG                  # BF16 with scales
    assert call(c, (7, None)) == L.EP_ERR_INVALID_ARG                 # no recv_src
    assert call(c, (0, FAKE + 8)) == L.EP_ERR_ALIGNMENT
    assert call(c, (8, FAKE + 2)) == L.EP_ERR_ALIGNMENT
    big = _cfg(T=1025).c()                                           # T * k > 8192
    assert call(big) == L.EP_ERR_UNSUPPORTED
    assert lib.ep_combine_ll(ctypes.byref(c), 0, FAKE, FAKE, FAKE, FAKE, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_combine_ll(ctypes.byref(c), 128, FAKE, FAKE, FAKE, None, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_combine_ll(ctypes.byref(c), 128, FAKE + 4, FAKE, FAKE, FAKE, None) == L.EP_ERR_ALIGNMENT
    z = _cfg(T=0).c()
    assert lib.ep_combine_ll(ctypes.byref(z), 4, None, None, None, None, None) == L.EP_OK


def test_rank_path_rejections():
    lib = ep.lib()
    c = _cfg().c()
    need = lib.ep_rank_layout_workspace_bytes(ctypes.byref(c))
    assert need > 0 and need % 256 == 0
    assert lib.ep_rank_layout_workspace_bytes(ctypes.byref(_cfg(H=100).c())) == 0
    a4 = [FAKE] * 4
    assert lib.ep_get_rank_layout(ctypes.byref(c), *a4, FAKE, FAKE, need - 1, None) == L.EP_ERR_WORKSPACE
    assert lib.ep_get_rank_layout(ctypes.byref(c), *a4, FAKE, None, need, None) == L.EP_ERR_WORKSPACE
    assert lib.ep_get_rank_layout(ctypes.byref(c), *a4, FAKE, FAKE + 128, need, None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_get_rank_layout(ctypes.byref(c), FAKE, None, FAKE, FAKE, FAKE, FAKE, need,
                                  None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_combine_rank_partial(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                       None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_combine_rank_partial(ctypes.byref(c), FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == L.EP_ERR_ALIGNMENT
    assert lib.ep_combine_ranks(ctypes.byref(c), FAKE, FAKE, None, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_combine_ranks(ctypes.byref(c), FAKE, FAKE + 2, FAKE, None) == L.EP_ERR_ALIGNMENT
    z = _cfg(T=0).c()
    assert lib.ep_combine_ranks(ctypes.byref(z), None, None, None, None) == L.EP_OK


def test_cu_range_stream_rejections():
    lib = ep.lib()
    h = ctypes.c_void_p()
    # rejected before any HIP call
    assert lib.ep_stream_create_cu_range(0, 0, ctypes.byref(h)) == L.EP_ERR_INVALID_ARG
    assert lib.ep_stream_create_cu_range(-1, 8, ctypes.byref(h)) == L.EP_ERR_INVALID_ARG
    assert lib.ep_stream_create_cu_range(0, 8, None) == L.EP_ERR_INVALID_ARG
    assert lib.ep_stream_destroy(None) == L.EP_ERR_INVALID_ARG


def test_binding_rejects_cpu_tensors():
    import torch
    w = W.TINY
    cfg = ep.Config.of(w)
    with pytest.raises(ValueError):
        ep.route(cfg, torch.zeros((w.T, w.E)))
