"""BSR block-sparse attention over a KV cache for AMD MI355X (gfx950).

The compute path is libbsa.so (hand-written HIP kernels behind the C ABI in
include/bsa.h); this package is its thin Python binding plus seeded
synthetic workloads.
"""
from .api import Plan, indexer_topk, merge_states, mla_rope_quantize_fp8  # noqa: F401

__all__ = ["Plan", "indexer_topk", "merge_states", "mla_rope_quantize_fp8"]
