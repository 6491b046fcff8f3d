"""Algorithmic byte accounting for the decode path (what the method must move).

Per token and KV head, K plus V is 2 * head_dim * elem_bytes bytes. This matches
the KV ledger of the TileLang tutorial ch. 18, section 2.5 (bytes per token per
layer = 2 * n_kv_heads * head_dim * b) and the decode-attention arithmetic
intensity of section 2.4 (AI = 2 * H_q / (H_kv * b) FLOP per byte). Nothing here
counts re-reads, split-KV partials or padding: those are overheads a kernel adds.

Used by bench.py for the achieved-bandwidth figures; pinned against the
tutorial's worked numbers in tests/test_roofline.py.
"""
from __future__ import annotations

import numpy as np

MI355X_HBM_GBPS = 8000.0          # published peak HBM3E bandwidth
BF16 = 2


def kv_bytes_per_token_layer(num_kv_heads: int, head_dim: int, elem_bytes: int = BF16) -> int:
    return 2 * num_kv_heads * head_dim * elem_bytes


def decode_attention_ai(num_q_heads: int, num_kv_heads: int, elem_bytes: int = BF16) -> float:
    """FLOP per KV byte of single-token decode attention (two contractions)."""
    return 2.0 * num_q_heads / (num_kv_heads * elem_bytes)


def dense_attention_bytes(context_lens, num_kv_heads: int, head_dim: int) -> int:
    return int(np.asarray(context_lens, dtype=np.int64).sum()) * kv_bytes_per_token_layer(
        num_kv_heads, head_dim)


def dense_attention_bytes_fp8(context_lens, num_kv_heads: int, head_dim: int) -> int:
    """K + V codes of every valid token (1 byte per element)."""
    return int(np.asarray(context_lens, dtype=np.int64).sum()) * kv_bytes_per_token_layer(
        num_kv_heads, head_dim, elem_bytes=1)


def write_bytes(slot_mapping, num_blocks: int, block_size: int, num_kv_heads: int,
                head_dim: int) -> int:
    """Read the new K/V rows and write them into the cache."""
    s = np.asarray(slot_mapping, dtype=np.int64)
    valid = int(((s >= 0) & (s < num_blocks * block_size)).sum())
    return valid * kv_bytes_per_token_layer(num_kv_heads, head_dim) * 2


def fused_write_bytes(slot_mapping, num_blocks: int, block_size: int, num_kv_heads: int,
                      head_dim: int) -> int:
    """The K/V write, plus per written token its block's min / max row: read when the
    token is not at row 0 of its block, always written."""
    s = np.asarray(slot_mapping, dtype=np.int64)
    s = s[(s >= 0) & (s < num_blocks * block_size)]
    row = num_kv_heads * head_dim * BF16
    folded = int((s % block_size != 0).sum())
    return write_bytes(s, num_blocks, block_size, num_kv_heads, head_dim) + folded * 2 * row \
        + int(s.size) * 2 * row


def metadata_step_bytes(context_lens, block_size: int, num_kv_heads: int, head_dim: int) -> int:
    """Read the valid K rows of each sequence's last block; write its min and max."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    live = ctx > 0
    last_rows = ctx[live] - (ctx[live] - 1) // block_size * block_size
    row = num_kv_heads * head_dim * BF16
    return int(last_rows.sum()) * row + int(live.sum()) * 2 * row


def metadata_full_bytes(context_lens, block_size: int, num_kv_heads: int, head_dim: int) -> int:
    ctx = np.asarray(context_lens, dtype=np.int64)
    nb = (ctx + block_size - 1) // block_size
    row = num_kv_heads * head_dim * BF16
    return int(ctx.sum()) * row + int(nb.sum()) * 2 * row


def select_bytes(context_lens, block_size: int, num_kv_heads: int, head_dim: int,
                 elem_bytes: int = BF16) -> int:
    """Scan the key min/max of every valid block of every (sequence, KV head)
    (elem_bytes 1: E4M3 code metadata)."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    nb = (ctx + block_size - 1) // block_size
    return int(nb.sum()) * num_kv_heads * 2 * head_dim * elem_bytes


def fused_write_bytes_fp8(slot_mapping, num_blocks: int, block_size: int, num_kv_heads: int,
                          head_dim: int) -> int:
    """The FP8 write (bf16 rows in, E4M3 codes out) with the code metadata fold: per
    written token its block's min / max code rows, read when the token is not at row 0
    of its block, always written."""
    s = np.asarray(slot_mapping, dtype=np.int64)
    s = s[(s >= 0) & (s < num_blocks * block_size)]
    row = num_kv_heads * head_dim          # bytes of one code row
    folded = int((s % block_size != 0).sum())
    return int(s.size) * (2 * row * BF16 + 2 * row) + folded * 2 * row + int(s.size) * 2 * row


def sparse_attention_bytes(topk_indices, context_lens, block_size: int, head_dim: int,
                           elem_bytes: int = BF16) -> int:
    """K + V of the valid tokens of every selected block, per KV head (elem_bytes 1:
    E4M3 caches)."""
    sel = np.asarray(topk_indices, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)[:, None, None]
    nb = (ctx + block_size - 1) // block_size
    ok = (sel >= 0) & (sel < nb)
    valid = np.clip(ctx - sel * block_size, 0, block_size)
    tokens = int(np.where(ok, valid, 0).sum())
    return tokens * 2 * head_dim * elem_bytes
