"""MI355X-native varlen chunked Gated Delta Rule prefill (libgdn_prefill).

``chunk_gated_delta_rule``, ``gated_delta_rule_decode`` and
``build_chunk_indices`` call the HIP kernels of the in-tree
``libgdn_prefill.so`` through its C ABI (include/gdn_prefill.h).
"""
from .api import (build_chunk_indices, chunk_gated_delta_rule,  # noqa: F401
                  gated_delta_rule_decode)

__all__ = ["chunk_gated_delta_rule", "gated_delta_rule_decode", "build_chunk_indices"]
