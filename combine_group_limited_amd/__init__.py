"""MI355X-native MoE routing, dispatch and combine (one GPU's share).

The computation lives in libep.so (hand-written HIP kernels for gfx950
behind the C ABI of include/ep.h); this package is its Python binding.
"""
from ._lib import EXPORTS, LIB_PATH, lib  # noqa: F401
from .api import (  # noqa: F401
    Config,
    CuRangeStream,
    EpError,
    combine,
    combine_ll,
    combine_rank_partial,
    combine_ranks,
    dispatch,
    dispatch_ll,
    get_layout,
    get_layout_static,
    get_rank_layout,
    layout_workspace_bytes,
    rank_layout_workspace_bytes,
    route,
    route_layout,
    route_layout_workspace_bytes,
    scores,
    validate,
)
