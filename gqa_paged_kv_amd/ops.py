"""torch-tensor front end of the gpkv C ABI (names follow include/gpkv.h).

Tensors must live on the GPU and be contiguous. bf16 tensors are torch.bfloat16;
block_tables / context_lens / topk indices are int32, slot_mapping is int64 and
attention outputs are float32. Every call is asynchronous on
torch.cuda.current_stream() (or the ``stream`` given).
"""
from __future__ import annotations

import torch

from ._lib import lib

__all__ = [
    "GpkvError", "reshape_and_cache", "reshape_and_cache_quest", "paged_attention_decode",
    "paged_attention_decode_append", "quest_decode_append", "quest_block_metadata",
    "quest_select_topk", "sparse_paged_attention_decode", "paged_attention_workspace_bytes",
    "quest_select_workspace_bytes", "sparse_attention_workspace_bytes", "split_tokens",
    "reshape_and_cache_fp8", "paged_attention_decode_fp8", "sparse_paged_attention_decode_fp8",
    "paged_attention_decode_fp8_append", "paged_attention_varlen",
    "paged_attention_varlen_workspace_bytes",
]


class GpkvError(RuntimeError):
    """A gpkv call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        self.status = status
        self.message = message
        name = lib().gpkv_status_string(status).decode()
        super().__init__(f"gpkv status {status} ({name}): {message}")


def _check(status: int) -> None:
    if status != 0:
        raise GpkvError(status, lib().gpkv_last_error_message().decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(name: str, t: torch.Tensor, dtype: torch.dtype, ndim: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {tuple(t.shape)})")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes: int, device, workspace: torch.Tensor | None) -> torch.Tensor:
    if workspace is not None:
        _dev("workspace", workspace, torch.uint8)
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _cache_dims(key_cache: torch.Tensor):
    NB, bs, Hkv, D = key_cache.shape
    return int(NB), int(bs), int(Hkv), int(D)


def split_tokens(batch: int, num_kv_heads: int, span_tokens: int) -> int:
    return int(lib().gpkv_split_tokens(batch, num_kv_heads, span_tokens))


def paged_attention_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                    max_context_len) -> int:
    return int(lib().gpkv_paged_attention_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len))


def quest_select_workspace_bytes(batch, num_kv_heads, max_blocks_per_seq) -> int:
    return int(lib().gpkv_quest_select_workspace_bytes(batch, num_kv_heads, max_blocks_per_seq))


def sparse_attention_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                     topk_blocks) -> int:
    return int(lib().gpkv_sparse_attention_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, block_size, topk_blocks))


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, *, stream=None) -> None:
    """Write key[i] / value[i] to the cache slot slot_mapping[i] (negative: skip)."""
    _dev("key_cache", key_cache, torch.bfloat16, 4)
    _dev("value_cache", value_cache, torch.bfloat16, 4)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    T = key.shape[0]
    if value_cache.shape != key_cache.shape or key.shape != (T, Hkv, D) or value.shape != key.shape \
            or slot_mapping.shape[0] != T:
        raise ValueError("reshape_and_cache: inconsistent shapes")
    _check(lib().gpkv_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping), T, Hkv, D,
        bs, NB, _stream(stream)))


def reshape_and_cache_quest(key, value, key_cache, value_cache, key_min, key_max, slot_mapping,
                            *, stream=None) -> None:
    """reshape_and_cache plus the incremental Quest key min / max of each written block."""
    _dev("key_cache", key_cache, torch.bfloat16, 4)
    _dev("value_cache", value_cache, torch.bfloat16, 4)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("key_min", key_min, torch.bfloat16, 3)
    _dev("key_max", key_max, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    T = key.shape[0]
    if value_cache.shape != key_cache.shape or key.shape != (T, Hkv, D) or value.shape != key.shape \
            or slot_mapping.shape[0] != T or key_min.shape != (NB, Hkv, D) \
            or key_max.shape != (NB, Hkv, D):
        raise ValueError("reshape_and_cache_quest: inconsistent shapes")
    _check(lib().gpkv_reshape_and_cache_quest(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(key_min), _ptr(key_max),
        _ptr(slot_mapping), T, Hkv, D, bs, NB, _stream(stream)))


def _attn_checks(query, key_cache, value_cache, block_tables, context_lens):
    _dev("query", query, torch.bfloat16, 3)
    _dev("key_cache", key_cache, torch.bfloat16, 4)
    _dev("value_cache", value_cache, torch.bfloat16, 4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    B, Hq, Dq = query.shape
    if value_cache.shape != key_cache.shape or Dq != D or block_tables.shape[0] != B \
            or context_lens.shape[0] != B:
        raise ValueError("inconsistent shapes between query, caches, block_tables, context_lens")
    return B, Hq, Hkv, D, bs, NB, int(block_tables.shape[1])


def paged_attention_decode(query, key_cache, value_cache, block_tables, context_lens, *,
                           max_context_len: int, scale: float, out=None, workspace=None,
                           stream=None) -> torch.Tensor:
    """Dense GQA paged decode attention; returns out [B, H_q, D] float32."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks(query, key_cache, value_cache, block_tables,
                                             context_lens)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_paged_attention_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), B, Hq, Hkv, D, bs, NB, MB, int(max_context_len), float(scale),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def paged_attention_decode_append(query, key, value, key_cache, value_cache, slot_mapping,
                                  block_tables, context_lens, *, max_context_len: int,
                                  scale: float, key_min=None, key_max=None, out=None,
                                  workspace=None, stream=None) -> torch.Tensor:
    """Decode append: writes token b of key / value (sequence b's newest token, at
    position context_lens[b] - 1) to slot_mapping[b] (with the Quest key min / max
    fold when key_min / key_max are given) and returns the dense attention over the
    contexts including it, out [B, H_q, D] float32 -- one call, two launches."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks(query, key_cache, value_cache, block_tables,
                                             context_lens)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape[0] != B:
        raise ValueError("paged_attention_decode_append: key / value / slot_mapping must hold "
                         "one token per sequence")
    if (key_min is None) != (key_max is None):
        raise ValueError("paged_attention_decode_append: key_min and key_max go together")
    if key_min is not None:
        _dev("key_min", key_min, torch.bfloat16, 3)
        _dev("key_max", key_max, torch.bfloat16, 3)
        if key_min.shape != (NB, Hkv, D) or key_max.shape != (NB, Hkv, D):
            raise ValueError("paged_attention_decode_append: inconsistent metadata shapes")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_paged_attention_decode_append(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
        _ptr(key_min) if key_min is not None else None,
        _ptr(key_max) if key_max is not None else None, _ptr(slot_mapping), _ptr(block_tables),
        _ptr(context_lens), B, Hq, Hkv, D, bs, NB, MB, int(max_context_len), float(scale),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def paged_attention_decode_noalloc(query, key_cache, value_cache, block_tables, context_lens,
                                   out, *, max_context_len: int, scale: float,
                                   stream=None) -> torch.Tensor:
    """Dense GQA paged decode attention without a workspace: the library's fixed device
    scratch array holds the partial rows (calls overlapping on one GPU race). ``out``
    [B, H_q, D] float32 is required, so the call allocates nothing."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks(query, key_cache, value_cache, block_tables,
                                             context_lens)
    _dev("out", out, torch.float32, 3)
    _check(lib().gpkv_paged_attention_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), B, Hq, Hkv, D, bs, NB, MB, int(max_context_len), float(scale),
        _stream(stream)))
    return out


def quest_block_metadata(key_cache, block_tables, context_lens, key_min, key_max, *,
                         max_context_len: int, last_block_only: bool = False,
                         stream=None) -> None:
    """Refresh per-block key min / max (all referenced blocks, or each last block)."""
    _dev("key_cache", key_cache, torch.bfloat16, 4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    _dev("key_min", key_min, torch.bfloat16, 3)
    _dev("key_max", key_max, torch.bfloat16, 3)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    B = int(context_lens.shape[0])
    if key_min.shape != (NB, Hkv, D) or key_max.shape != (NB, Hkv, D) \
            or block_tables.shape[0] != B:
        raise ValueError("quest_block_metadata: inconsistent shapes")
    _check(lib().gpkv_quest_block_metadata(
        _ptr(key_min), _ptr(key_max), _ptr(key_cache), _ptr(block_tables), _ptr(context_lens), B,
        Hkv, D, bs, NB, int(block_tables.shape[1]), int(max_context_len),
        1 if last_block_only else 0, _stream(stream)))


def quest_select_topk(query, key_min, key_max, block_tables, context_lens, *, block_size: int,
                      topk_blocks: int, max_context_len: int, out=None, workspace=None,
                      stream=None) -> torch.Tensor:
    """Quest block scores + Top-K; returns [B, H_kv, topk_blocks] int32 (ascending, -1 pad)."""
    _dev("query", query, torch.bfloat16, 3)
    _dev("key_min", key_min, torch.bfloat16, 3)
    _dev("key_max", key_max, torch.bfloat16, 3)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    NB, Hkv, D = (int(x) for x in key_min.shape)
    B, Hq, Dq = query.shape
    MB = int(block_tables.shape[1])
    if key_max.shape != key_min.shape or Dq != D or block_tables.shape[0] != B \
            or context_lens.shape[0] != B:
        raise ValueError("quest_select_topk: inconsistent shapes")
    if out is None:
        out = torch.empty((B, Hkv, int(topk_blocks)), dtype=torch.int32, device=query.device)
    _dev("out", out, torch.int32, 3)
    ws = _workspace(quest_select_workspace_bytes(B, Hkv, MB), query.device, workspace)
    _check(lib().gpkv_quest_select_topk(
        _ptr(out), _ptr(query), _ptr(key_min), _ptr(key_max), _ptr(block_tables),
        _ptr(context_lens), B, Hq, Hkv, D, int(block_size), NB, MB, int(max_context_len),
        int(topk_blocks), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def sparse_paged_attention_decode(query, key_cache, value_cache, block_tables, context_lens,
                                  topk_indices, *, max_context_len: int, scale: float, out=None,
                                  workspace=None, stream=None) -> torch.Tensor:
    """Exact attention over the selected logical blocks; returns [B, H_q, D] float32."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks(query, key_cache, value_cache, block_tables,
                                             context_lens)
    _dev("topk_indices", topk_indices, torch.int32, 3)
    if topk_indices.shape[0] != B or topk_indices.shape[1] != Hkv:
        raise ValueError("sparse_paged_attention_decode: topk_indices must be [B, H_kv, K]")
    K = int(topk_indices.shape[2])
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = sparse_attention_workspace_bytes(B, Hq, Hkv, D, bs, K)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_sparse_paged_attention_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(topk_indices), B, Hq, Hkv, D, bs, NB, MB, int(max_context_len),
        K, float(scale), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def quest_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                 max_blocks_per_seq, topk_blocks) -> int:
    return int(lib().gpkv_quest_decode_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                       head_dim, block_size, max_blocks_per_seq,
                                                       topk_blocks))


def quest_decode(query, key_cache, value_cache, key_min, key_max, block_tables, context_lens, *,
                 topk_blocks: int, max_context_len: int, scale: float, out=None, topk_out=None,
                 workspace=None, stream=None):
    """Quest selection and sparse attention in one call; returns (out [B, H_q, D] float32,
    topk_indices [B, H_kv, topk_blocks] int32), the results of quest_select_topk followed
    by sparse_paged_attention_decode."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks(query, key_cache, value_cache, block_tables,
                                             context_lens)
    _dev("key_min", key_min, torch.bfloat16, 3)
    _dev("key_max", key_max, torch.bfloat16, 3)
    if key_min.shape != key_max.shape or tuple(key_min.shape) != (NB, Hkv, D):
        raise ValueError("quest_decode: key_min / key_max must be [num_blocks, H_kv, D]")
    K = int(topk_blocks)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    if topk_out is None:
        topk_out = torch.empty((B, Hkv, K), dtype=torch.int32, device=query.device)
    _dev("out", out, torch.float32, 3)
    _dev("topk_out", topk_out, torch.int32, 3)
    if tuple(topk_out.shape) != (B, Hkv, K):
        raise ValueError("quest_decode: topk_out must be [B, H_kv, topk_blocks]")
    need = quest_decode_workspace_bytes(B, Hq, Hkv, D, bs, MB, K)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_quest_decode(
        _ptr(out), _ptr(topk_out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _ptr(key_min), _ptr(key_max), _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, bs,
        NB, MB, int(max_context_len), K, float(scale), _ptr(ws), ws.numel(), _stream(stream)))
    return out, topk_out


def quest_decode_append(query, key, value, key_cache, value_cache, key_min, key_max,
                        slot_mapping, block_tables, context_lens, *, topk_blocks: int,
                        max_context_len: int, scale: float, out=None, topk_out=None,
                        workspace=None, stream=None):
    """The Quest step with its cache write: reshape_and_cache_quest of token b of key /
    value (sequence b's newest token) at slot_mapping[b], then quest_decode over the
    written cache; returns (out, topk_indices) as quest_decode."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks(query, key_cache, value_cache, block_tables,
                                             context_lens)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    _dev("key_min", key_min, torch.bfloat16, 3)
    _dev("key_max", key_max, torch.bfloat16, 3)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape[0] != B:
        raise ValueError("quest_decode_append: key / value / slot_mapping must hold one token "
                         "per sequence")
    if key_min.shape != key_max.shape or tuple(key_min.shape) != (NB, Hkv, D):
        raise ValueError("quest_decode_append: key_min / key_max must be [num_blocks, H_kv, D]")
    K = int(topk_blocks)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    if topk_out is None:
        topk_out = torch.empty((B, Hkv, K), dtype=torch.int32, device=query.device)
    _dev("out", out, torch.float32, 3)
    _dev("topk_out", topk_out, torch.int32, 3)
    if tuple(topk_out.shape) != (B, Hkv, K):
        raise ValueError("quest_decode_append: topk_out must be [B, H_kv, topk_blocks]")
    need = quest_decode_workspace_bytes(B, Hq, Hkv, D, bs, MB, K)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_quest_decode_append(
        _ptr(out), _ptr(topk_out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache),
        _ptr(value_cache), _ptr(key_min), _ptr(key_max), _ptr(slot_mapping), _ptr(block_tables),
        _ptr(context_lens), B, Hq, Hkv, D, bs, NB, MB, int(max_context_len), K, float(scale),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out, topk_out


# ---------------------------------------------------------------------------
# FP8 (E4M3) caches: uint8 codes, float32 scale per KV head for K and for V
# ---------------------------------------------------------------------------

def _scales(k_scale, v_scale, Hkv):
    _dev("k_scale", k_scale, torch.float32, 1)
    _dev("v_scale", v_scale, torch.float32, 1)
    if k_scale.shape[0] != Hkv or v_scale.shape[0] != Hkv:
        raise ValueError("k_scale / v_scale must have num_kv_heads entries")


def reshape_and_cache_fp8(key, value, key_cache, value_cache, k_scale, v_scale, slot_mapping, *,
                          stream=None) -> None:
    """Quantise key[i] / value[i] to E4M3 with the per-head scales into slot slot_mapping[i]."""
    _dev("key_cache", key_cache, torch.uint8, 4)
    _dev("value_cache", value_cache, torch.uint8, 4)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    _scales(k_scale, v_scale, Hkv)
    T = key.shape[0]
    if value_cache.shape != key_cache.shape or key.shape != (T, Hkv, D) or value.shape != key.shape \
            or slot_mapping.shape[0] != T:
        raise ValueError("reshape_and_cache_fp8: inconsistent shapes")
    _check(lib().gpkv_reshape_and_cache_fp8(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(slot_mapping), T, Hkv, D, bs, NB, _stream(stream)))


def _attn_checks_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens):
    _dev("query", query, torch.bfloat16, 3)
    _dev("key_cache", key_cache, torch.uint8, 4)
    _dev("value_cache", value_cache, torch.uint8, 4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    _scales(k_scale, v_scale, Hkv)
    B, Hq, Dq = query.shape
    if value_cache.shape != key_cache.shape or Dq != D or block_tables.shape[0] != B \
            or context_lens.shape[0] != B:
        raise ValueError("inconsistent shapes between query, caches, block_tables, context_lens")
    return B, Hq, Hkv, D, bs, NB, int(block_tables.shape[1])


def paged_attention_decode_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables,
                               context_lens, *, max_context_len: int, scale: float, out=None,
                               workspace=None, stream=None) -> torch.Tensor:
    """Dense GQA paged decode attention over E4M3 caches; returns [B, H_q, D] float32."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                                 block_tables, context_lens)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_paged_attention_decode_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, bs, NB, MB, int(max_context_len),
        float(scale), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def paged_attention_decode_fp8_append(query, key, value, key_cache, value_cache, k_scale,
                                      v_scale, slot_mapping, block_tables, context_lens, *,
                                      max_context_len: int, scale: float, out=None,
                                      workspace=None, stream=None) -> torch.Tensor:
    """The FP8 dense step in one call: token b of key / value (bf16, sequence b's newest
    token) quantised into the E4M3 caches at slot_mapping[b], and the dense attention
    over the written caches; returns [B, H_q, D] float32."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                                 block_tables, context_lens)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape[0] != B:
        raise ValueError("paged_attention_decode_fp8_append: key / value / slot_mapping must hold "
                         "one token per sequence")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_paged_attention_decode_fp8_append(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens),
        B, Hq, Hkv, D, bs, NB, MB, int(max_context_len), float(scale), _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def sparse_paged_attention_decode_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                      block_tables, context_lens, topk_indices, *,
                                      max_context_len: int, scale: float, out=None,
                                      workspace=None, stream=None) -> torch.Tensor:
    """Attention over the selected logical blocks of E4M3 caches; returns [B, H_q, D] float32."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                                 block_tables, context_lens)
    _dev("topk_indices", topk_indices, torch.int32, 3)
    if topk_indices.shape[0] != B or topk_indices.shape[1] != Hkv:
        raise ValueError("sparse_paged_attention_decode_fp8: topk_indices must be [B, H_kv, K]")
    K = int(topk_indices.shape[2])
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = sparse_attention_workspace_bytes(B, Hq, Hkv, D, bs, K)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_sparse_paged_attention_decode_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), _ptr(topk_indices), B, Hq, Hkv, D, bs, NB, MB,
        int(max_context_len), K, float(scale), _ptr(ws), ws.numel(), _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# Quest over E4M3 caches: the metadata holds uint8 codes of the key code extremes
# ---------------------------------------------------------------------------

def _meta_fp8(fn, key_min, key_max, NB, Hkv, D):
    _dev("key_min", key_min, torch.uint8, 3)
    _dev("key_max", key_max, torch.uint8, 3)
    if key_min.shape != key_max.shape or tuple(key_min.shape) != (NB, Hkv, D):
        raise ValueError(f"{fn}: key_min / key_max must be [num_blocks, H_kv, D] uint8")


def quest_block_metadata_fp8(key_cache, block_tables, context_lens, key_min, key_max, *,
                             max_context_len: int, last_block_only: bool = False,
                             stream=None) -> None:
    """quest_block_metadata over an E4M3 key cache: codes of each channel's extremes."""
    _dev("key_cache", key_cache, torch.uint8, 4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    _meta_fp8("quest_block_metadata_fp8", key_min, key_max, NB, Hkv, D)
    B = int(context_lens.shape[0])
    if block_tables.shape[0] != B:
        raise ValueError("quest_block_metadata_fp8: inconsistent shapes")
    _check(lib().gpkv_quest_block_metadata_fp8(
        _ptr(key_min), _ptr(key_max), _ptr(key_cache), _ptr(block_tables), _ptr(context_lens), B,
        Hkv, D, bs, NB, int(block_tables.shape[1]), int(max_context_len),
        1 if last_block_only else 0, _stream(stream)))


def reshape_and_cache_fp8_quest(key, value, key_cache, value_cache, k_scale, v_scale, key_min,
                                key_max, slot_mapping, *, stream=None) -> None:
    """reshape_and_cache_fp8 plus the fold of each written key row's codes into its
    block's code metadata."""
    _dev("key_cache", key_cache, torch.uint8, 4)
    _dev("value_cache", value_cache, torch.uint8, 4)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    _scales(k_scale, v_scale, Hkv)
    _meta_fp8("reshape_and_cache_fp8_quest", key_min, key_max, NB, Hkv, D)
    T = key.shape[0]
    if value_cache.shape != key_cache.shape or key.shape != (T, Hkv, D) or value.shape != key.shape \
            or slot_mapping.shape[0] != T:
        raise ValueError("reshape_and_cache_fp8_quest: inconsistent shapes")
    _check(lib().gpkv_reshape_and_cache_fp8_quest(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(key_min), _ptr(key_max), _ptr(slot_mapping), T, Hkv, D, bs, NB, _stream(stream)))


def quest_select_topk_fp8(query, key_min, key_max, block_tables, context_lens, *, block_size: int,
                          topk_blocks: int, max_context_len: int, out=None, workspace=None,
                          stream=None) -> torch.Tensor:
    """quest_select_topk over E4M3 code metadata; returns [B, H_kv, topk_blocks] int32."""
    _dev("query", query, torch.bfloat16, 3)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    NB, Hkv, D = (int(x) for x in key_min.shape)
    _meta_fp8("quest_select_topk_fp8", key_min, key_max, NB, Hkv, D)
    B, Hq, Dq = query.shape
    MB = int(block_tables.shape[1])
    if Dq != D or block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("quest_select_topk_fp8: inconsistent shapes")
    if out is None:
        out = torch.empty((B, Hkv, int(topk_blocks)), dtype=torch.int32, device=query.device)
    _dev("out", out, torch.int32, 3)
    ws = _workspace(quest_select_workspace_bytes(B, Hkv, MB), query.device, workspace)
    _check(lib().gpkv_quest_select_topk_fp8(
        _ptr(out), _ptr(query), _ptr(key_min), _ptr(key_max), _ptr(block_tables),
        _ptr(context_lens), B, Hq, Hkv, D, int(block_size), NB, MB, int(max_context_len),
        int(topk_blocks), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def _quest_outputs(fn, query, B, Hq, Hkv, D, K, out, topk_out):
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    if topk_out is None:
        topk_out = torch.empty((B, Hkv, K), dtype=torch.int32, device=query.device)
    _dev("out", out, torch.float32, 3)
    _dev("topk_out", topk_out, torch.int32, 3)
    if tuple(topk_out.shape) != (B, Hkv, K):
        raise ValueError(f"{fn}: topk_out must be [B, H_kv, topk_blocks]")
    return out, topk_out


def quest_decode_fp8(query, key_cache, value_cache, k_scale, v_scale, key_min, key_max,
                     block_tables, context_lens, *, topk_blocks: int, max_context_len: int,
                     scale: float, out=None, topk_out=None, workspace=None, stream=None):
    """quest_decode over E4M3 caches and code metadata; returns (out, topk_indices) as
    quest_select_topk_fp8 followed by sparse_paged_attention_decode_fp8."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                                 block_tables, context_lens)
    _meta_fp8("quest_decode_fp8", key_min, key_max, NB, Hkv, D)
    K = int(topk_blocks)
    out, topk_out = _quest_outputs("quest_decode_fp8", query, B, Hq, Hkv, D, K, out, topk_out)
    ws = _workspace(quest_decode_workspace_bytes(B, Hq, Hkv, D, bs, MB, K), query.device,
                    workspace)
    _check(lib().gpkv_quest_decode_fp8(
        _ptr(out), _ptr(topk_out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(key_min), _ptr(key_max), _ptr(block_tables), _ptr(context_lens), B,
        Hq, Hkv, D, bs, NB, MB, int(max_context_len), K, float(scale), _ptr(ws), ws.numel(),
        _stream(stream)))
    return out, topk_out


def quest_decode_fp8_append(query, key, value, key_cache, value_cache, k_scale, v_scale, key_min,
                            key_max, slot_mapping, block_tables, context_lens, *,
                            topk_blocks: int, max_context_len: int, scale: float, out=None,
                            topk_out=None, workspace=None, stream=None):
    """The FP8 Quest step with its cache write: reshape_and_cache_fp8_quest of token b of
    key / value (bf16, sequence b's newest token) at slot_mapping[b], then
    quest_decode_fp8 over the written caches; returns (out, topk_indices)."""
    B, Hq, Hkv, D, bs, NB, MB = _attn_checks_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                                 block_tables, context_lens)
    _dev("key", key, torch.bfloat16, 3)
    _dev("value", value, torch.bfloat16, 3)
    _dev("slot_mapping", slot_mapping, torch.int64, 1)
    _meta_fp8("quest_decode_fp8_append", key_min, key_max, NB, Hkv, D)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape[0] != B:
        raise ValueError("quest_decode_fp8_append: key / value / slot_mapping must hold one "
                         "token per sequence")
    K = int(topk_blocks)
    out, topk_out = _quest_outputs("quest_decode_fp8_append", query, B, Hq, Hkv, D, K, out,
                                   topk_out)
    ws = _workspace(quest_decode_workspace_bytes(B, Hq, Hkv, D, bs, MB, K), query.device,
                    workspace)
    _check(lib().gpkv_quest_decode_fp8_append(
        _ptr(out), _ptr(topk_out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache),
        _ptr(value_cache), _ptr(k_scale), _ptr(v_scale), _ptr(key_min), _ptr(key_max),
        _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, bs, NB, MB,
        int(max_context_len), K, float(scale), _ptr(ws), ws.numel(), _stream(stream)))
    return out, topk_out


# ---------------------------------------------------------------------------
# Multi-token queries (varlen, causal mask aligned to the right)
# ---------------------------------------------------------------------------

def paged_attention_varlen_workspace_bytes(batch, total_q, max_q_len, num_q_heads, num_kv_heads,
                                           head_dim, block_size, max_context_len) -> int:
    return int(lib().gpkv_paged_attention_varlen_workspace_bytes(
        batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size,
        max_context_len))


def paged_attention_varlen(query, key_cache, value_cache, block_tables, context_lens, cu_seqlens_q,
                           *, max_q_len: int, max_context_len: int, scale: float, out=None,
                           workspace=None, stream=None) -> torch.Tensor:
    """Attention of every query row of a flattened multi-token batch; returns
    [total_q, H_q, D] float32. Row j of sequence b sees positions
    <= context_lens[b] - q_len_b + j."""
    _dev("query", query, torch.bfloat16, 3)
    _dev("key_cache", key_cache, torch.bfloat16, 4)
    _dev("value_cache", value_cache, torch.bfloat16, 4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    _dev("cu_seqlens_q", cu_seqlens_q, torch.int32, 1)
    NB, bs, Hkv, D = _cache_dims(key_cache)
    UQ, Hq, Dq = query.shape
    B = int(context_lens.shape[0])
    if value_cache.shape != key_cache.shape or Dq != D or block_tables.shape[0] != B \
            or cu_seqlens_q.shape[0] != B + 1:
        raise ValueError("paged_attention_varlen: inconsistent shapes")
    if out is None:
        out = torch.empty((UQ, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = paged_attention_varlen_workspace_bytes(B, UQ, max_q_len, Hq, Hkv, D, bs,
                                                  max_context_len)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_paged_attention_varlen(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(cu_seqlens_q), B, UQ, int(max_q_len), Hq, Hkv, D, bs, NB,
        int(block_tables.shape[1]), int(max_context_len), float(scale), _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def paged_attention_varlen_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables,
                               context_lens, cu_seqlens_q, *, max_q_len: int, max_context_len: int,
                               scale: float, out=None, workspace=None, stream=None) -> torch.Tensor:
    """paged_attention_varlen over E4M3 caches (uint8 codes, float32 scale per KV head);
    returns [total_q, H_q, D] float32."""
    _dev("query", query, torch.bfloat16, 3)
    _dev("key_cache", key_cache, torch.uint8, 4)
    _dev("value_cache", value_cache, torch.uint8, 4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    _dev("cu_seqlens_q", cu_seqlens_q, torch.int32, 1)
    NB, bs, Hkv, D = (int(x) for x in key_cache.shape)
    _scales(k_scale, v_scale, Hkv)
    UQ, Hq, Dq = query.shape
    B = int(context_lens.shape[0])
    if value_cache.shape != key_cache.shape or Dq != D or block_tables.shape[0] != B \
            or cu_seqlens_q.shape[0] != B + 1:
        raise ValueError("paged_attention_varlen_fp8: inconsistent shapes")
    if out is None:
        out = torch.empty((UQ, Hq, D), dtype=torch.float32, device=query.device)
    _dev("out", out, torch.float32, 3)
    need = paged_attention_varlen_workspace_bytes(B, UQ, max_q_len, Hq, Hkv, D, bs,
                                                  max_context_len)
    ws = _workspace(need, query.device, workspace)
    _check(lib().gpkv_paged_attention_varlen_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), _ptr(cu_seqlens_q), B, UQ, int(max_q_len), Hq,
        Hkv, D, bs, NB, int(block_tables.shape[1]), int(max_context_len), float(scale), _ptr(ws),
        ws.numel(), _stream(stream)))
    return out
