"""MI355X-native neighbourhood attention for one context-parallel rank.

A query shard attends over its collected K/V neighbourhood with per-document
causal masking (packed doc ids, pad id 0), bottom-right alignment, an optional
left window and GQA.  Everything runs in the HIP library ``libnbattn.so``
(include/nbattn.h); this package is its thin Python binding.
"""
from .api import (BwdResult, ChunkSaved, KvChunk, NeighbourhoodAttention, OwnerTable, Saved, Segments, attn_bwd,
                  attn_bwd_chunks, attn_fwd, attn_fwd_chunks, neighbourhood_attention, ring_window_chunks,
                  segment_build)

__all__ = ["segment_build", "attn_fwd", "attn_bwd", "Segments", "OwnerTable", "Saved", "BwdResult",
           "NeighbourhoodAttention", "neighbourhood_attention", "KvChunk", "ChunkSaved", "attn_fwd_chunks",
           "attn_bwd_chunks", "ring_window_chunks"]
