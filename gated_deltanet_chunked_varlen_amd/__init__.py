"""MI355X-native varlen chunked Gated Delta Rule prefill (libgdn_prefill).

``chunk_gated_delta_rule`` (with ``use_cp`` for context parallelism within
the GPU), ``chunk_gated_delta_rule_noalloc``, ``gated_delta_rule_decode`` and
``build_chunk_indices`` call the HIP kernels of the in-tree
``libgdn_prefill.so`` through its C ABI (include/gdn_prefill.h);
``PrefillGraphs`` replays one captured HIP graph per set of buffer addresses.
"""
from .api import (PrefillGraphs, build_chunk_indices, chunk_gated_delta_rule,  # noqa: F401
                  chunk_gated_delta_rule_noalloc, clear_workspace_cache,
                  gated_delta_rule_decode)

__all__ = ["chunk_gated_delta_rule", "chunk_gated_delta_rule_noalloc", "gated_delta_rule_decode",
           "build_chunk_indices", "PrefillGraphs", "clear_workspace_cache"]
