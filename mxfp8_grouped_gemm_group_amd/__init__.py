"""MI355X-native fused MXFP8 grouped-matmul + finalize-routing (MoE combine).

The operator runs in libgfr.so (HIP kernels for gfx950, C ABI in
include/gfr.h); this package is its thin Python binding plus the seeded input
generators (``workloads``).  The library is loaded on first use and its absence
is an error: there is no fallback implementation.
"""
from ._binding import (DEV_BAD_GROUP_LIST, DEV_BAD_ROW_INDEX, GfrError, gemm1_swiglu_quant,
                       gmm_finalize_routing, gmm_finalize_routing_det_noalloc, load_library,
                       status_string, w4a8_finalize_routing, workspace_size)

__all__ = ["gmm_finalize_routing", "gmm_finalize_routing_det_noalloc", "gemm1_swiglu_quant",
           "w4a8_finalize_routing", "workspace_size", "status_string", "load_library",
           "GfrError", "DEV_BAD_GROUP_LIST", "DEV_BAD_ROW_INDEX"]
