"""MI355X (gfx950) MoE route-count / dispatch / combine.

The compute path lives in libmoe_route.so (hand-written HIP kernels behind a
C ABI, declared in include/moe_route.h); this package is its thin Python
binding.  Import is cheap: the library is loaded on first use and its absence
raises instead of falling back to anything else.
"""
from ._lib import (DedupOut, DedupPlan, DispatchOut, MoeError, combine, combine_fp4, combine_fp8,
                   copy16,
                   dedup_dispatch, dispatch, dispatch_noalloc, dispatch_prequant, dispatch_replay, fp8_dequant,
                   geometry, load, route_count, version, workspace, workspace_size)

__all__ = ["DedupOut", "DedupPlan", "DispatchOut", "MoeError", "combine", "combine_fp4",
           "combine_fp8", "copy16",
           "dedup_dispatch", "dispatch", "dispatch_noalloc", "dispatch_prequant", "dispatch_replay", "fp8_dequant",
           "geometry", "load", "route_count", "version", "workspace", "workspace_size"]
