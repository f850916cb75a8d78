"""ctypes loader for libep.so (the C ABI of include/ep.h).

torch is imported first so that the HIP runtime torch ships is the one in
the process; libep.so links libamdhip64.so.7 by SONAME and binds to it.
If libep.so is missing, or was built from other sources than the current
ones (a content hash recorded at build time), it is rebuilt with hipcc, and
without hipcc the load is refused; if it cannot be loaded the import fails:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import threading

import torch  # noqa: F401  (loads torch's HIP runtime before libep.so)

from . import build as _build

LIB_PATH = _build.LIB_PATH

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_ALIGNMENT = -2
EP_ERR_UNSUPPORTED = -3
EP_ERR_WORKSPACE = -4
EP_ERR_HIP = -5
EP_ERR_SCRATCH_LIMIT = -6

# bytes of the device array ep_get_layout_static uses as its scratch
EP_STATIC_SCRATCH_BYTES = 1 << 20

EP_RECV_FP8_E4M3 = 0
EP_RECV_BF16 = 1

# every function include/ep.h declares
EXPORTS = (
    "ep_abi_version",
    "ep_strerror",
    "ep_last_hip_error",
    "ep_validate_config",
    "ep_route",
    "ep_scores",
    "ep_layout_workspace_bytes",
    "ep_get_layout",
    "ep_get_layout_static",
    "ep_route_layout_workspace_bytes",
    "ep_route_layout",
    "ep_dispatch",
    "ep_combine",
    "ep_dispatch_ll",
    "ep_combine_ll",
    "ep_rank_layout_workspace_bytes",
    "ep_get_rank_layout",
    "ep_combine_rank_partial",
    "ep_combine_ranks",
    "ep_stream_create_cu_range",
    "ep_stream_destroy",
)


class EpConfig(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("topk_groups", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("group_score_topm", ctypes.c_int32),
    ]


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libep.so with argument types declared."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _build.is_stale():
            if not _build.hipcc_available():
                raise RuntimeError("%s is missing or was built from other sources than those in %s, "
                                   "and hipcc is not available to rebuild it" % (LIB_PATH, _build.CSRC))
            print("libep.so is missing or out of date: rebuilding", flush=True)
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        C = ctypes.POINTER(EpConfig)
        I = ctypes.c_int
        L.ep_abi_version.argtypes = []
        L.ep_abi_version.restype = I
        L.ep_strerror.argtypes = [I]
        L.ep_strerror.restype = ctypes.c_char_p
        L.ep_last_hip_error.argtypes = []
        L.ep_last_hip_error.restype = I
        L.ep_validate_config.argtypes = [C]
        L.ep_validate_config.restype = I
        L.ep_route.argtypes = [C, P, P, P, P]
        L.ep_route.restype = I
        L.ep_scores.argtypes = [C, P, P, P]
        L.ep_scores.restype = I
        L.ep_layout_workspace_bytes.argtypes = [C]
        L.ep_layout_workspace_bytes.restype = ctypes.c_size_t
        L.ep_get_layout.argtypes = [C, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.ep_get_layout.restype = I
        L.ep_get_layout_static.argtypes = [C, P, P, P, P, P, P, P]
        L.ep_get_layout_static.restype = I
        L.ep_route_layout_workspace_bytes.argtypes = [C]
        L.ep_route_layout_workspace_bytes.restype = ctypes.c_size_t
        L.ep_route_layout.argtypes = [C, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.ep_route_layout.restype = I
        L.ep_dispatch.argtypes = [C, P, P, I, P, P, P]
        L.ep_dispatch.restype = I
        L.ep_combine.argtypes = [C, P, P, P, P, P]
        L.ep_combine.restype = I
        I32 = ctypes.c_int32
        L.ep_dispatch_ll.argtypes = [C, P, P, I32, I, P, P, P, P, P, P]
        L.ep_dispatch_ll.restype = I
        L.ep_combine_ll.argtypes = [C, I32, P, P, P, P, P]
        L.ep_combine_ll.restype = I
        L.ep_rank_layout_workspace_bytes.argtypes = [C]
        L.ep_rank_layout_workspace_bytes.restype = ctypes.c_size_t
        L.ep_get_rank_layout.argtypes = [C, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.ep_get_rank_layout.restype = I
        L.ep_combine_rank_partial.argtypes = [C, P, P, P, P, P, P, P]
        L.ep_combine_rank_partial.restype = I
        L.ep_combine_ranks.argtypes = [C, P, P, P, P]
        L.ep_combine_ranks.restype = I
        L.ep_stream_create_cu_range.argtypes = [I, I, ctypes.POINTER(P)]
        L.ep_stream_create_cu_range.restype = I
        L.ep_stream_destroy.argtypes = [P]
        L.ep_stream_destroy.restype = I
        _lib = L
        return _lib
