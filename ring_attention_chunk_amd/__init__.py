"""MI355X (gfx950) ring attention on one device's share: HIP kernels behind a C ABI.

``attention_chunk_stats``, ``merge_chunk_stats``, ``ring_attention`` and
``ring_attention_backward`` call the HIP library through ctypes (see
``api.py``); ``workloads`` builds the seeded
synthetic shares used by the tests and the benchmark.
"""

from .api import (
    EXPORTS,
    RingAttentionError,
    attention_chunk_stats,
    load_library,
    merge_chunk_stats,
    ring_attention,
    ring_attention_backward,
    ring_attention_block_sparse,
)

__all__ = [
    "EXPORTS",
    "RingAttentionError",
    "attention_chunk_stats",
    "load_library",
    "merge_chunk_stats",
    "ring_attention",
    "ring_attention_backward",
    "ring_attention_block_sparse",
]
