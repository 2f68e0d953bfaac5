"""MI355X-native varlen chunked Gated Delta Rule prefill (libgdn_prefill).

``chunk_gated_delta_rule`` and ``build_chunk_indices`` call the HIP kernels of
the in-tree ``libgdn_prefill.so`` through its C ABI (include/gdn_prefill.h).
"""
from .api import build_chunk_indices, chunk_gated_delta_rule  # noqa: F401

__all__ = ["chunk_gated_delta_rule", "build_chunk_indices"]
