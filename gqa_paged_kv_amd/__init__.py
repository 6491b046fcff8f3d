"""Paged GQA decode attention for AMD MI355X (gfx950): a thin torch binding over libgpkv.so.

Every function here checks tensor dtypes, devices and shapes, allocates the
workspace with torch's caching allocator when none is given, and calls the C ABI
of include/gpkv.h on torch's current HIP stream. All arithmetic runs in the HIP
kernels; there is no CPU or PyTorch fallback.
"""
from .ops import (GpkvError, paged_attention_decode, paged_attention_workspace_bytes,
                  quest_block_metadata, quest_select_topk, quest_select_workspace_bytes,
                  reshape_and_cache, reshape_and_cache_quest, sparse_attention_workspace_bytes,
                  sparse_paged_attention_decode, split_tokens, reshape_and_cache_fp8,
                  paged_attention_decode_fp8, sparse_paged_attention_decode_fp8,
                  paged_attention_varlen, paged_attention_varlen_workspace_bytes, quest_decode,
                  quest_decode_workspace_bytes, paged_attention_varlen_fp8,
                  paged_attention_decode_noalloc, paged_attention_decode_append,
                  quest_decode_append, paged_attention_decode_fp8_append,
                  quest_block_metadata_fp8, reshape_and_cache_fp8_quest, quest_select_topk_fp8,
                  quest_decode_fp8, quest_decode_fp8_append)

__all__ = [
    "GpkvError", "reshape_and_cache", "reshape_and_cache_quest", "paged_attention_decode",
    "quest_block_metadata",
    "quest_select_topk", "sparse_paged_attention_decode", "paged_attention_workspace_bytes",
    "quest_select_workspace_bytes", "sparse_attention_workspace_bytes", "split_tokens",
    "reshape_and_cache_fp8", "paged_attention_decode_fp8", "sparse_paged_attention_decode_fp8",
    "paged_attention_varlen", "paged_attention_varlen_workspace_bytes", "quest_decode",
    "quest_decode_workspace_bytes", "paged_attention_varlen_fp8", "paged_attention_decode_noalloc",
    "paged_attention_decode_append", "quest_decode_append", "paged_attention_decode_fp8_append",
    "quest_block_metadata_fp8", "reshape_and_cache_fp8_quest", "quest_select_topk_fp8",
    "quest_decode_fp8", "quest_decode_fp8_append",
]
