"""Seeded synthetic inputs for paged GQA decode attention.

This module only *draws* inputs; it holds none of the attention, cache-write or
Quest arithmetic. Both the CPU oracle (``oracle/``) and the HIP path read the
arrays it returns, so they see bit-identical inputs.

Every floating-point tensor is returned as raw bfloat16 bit patterns
(``numpy.uint16``), obtained from float32 normal samples by round-to-nearest-even.
Index tensors are int32 (block tables, context lengths) and int64 (slot mapping).

The five workloads follow the shapes the pages use for decode (Qwen2.5-7B head
shape: 28 query heads, 4 KV heads, head_dim 128 -- TileLang tutorial ch. 18,
sections 2.4-2.6) and the problem statement of the Ascend kernel-to-serving write-up
(sections "ReshapeAndCache", "GQA Paged Attention", "Quest Sparse Attention",
"extreme sequence length"). Where the pages give no distribution, the recipe below
is our own choice; it is fixed by the seed and documented per workload.

Workloads by number: 1 tiny GQA decode (B = 2, contexts 37 and 80); 2 Qwen-shaped
dense decode (B = 32, block size 128); 3 the ~8K-average ragged batch, dense vs Quest
(B = 64, block size 16); 4 four 40960-token sequences; 5 a ragged 256-sequence batch
with 8 KV heads.

Draw order for every workload (one ``numpy.random.default_rng(seed)`` stream):
  1. context_lens  2. block permutation  3. pool K / V  4. query
  5. new K / V and slot_mapping  6. Quest key offsets (the 8K-average batch only)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "make", "bf16_bits", "CONFIG_NAMES", "shape_summary"]

CONFIG_NAMES = {
    1: "tiny_gqa_b2_hq4_hkv1_d64_bs16",
    2: "qwen7b_dense_b32_hq28_hkv4_d128_bs128_ctx1k-8k",
    3: "long8k_dense_vs_quest_b64_hq28_hkv4_d128_bs16_k64",
    4: "extreme_40960_b4_hq28_hkv4_d128_bs16_k256",
    5: "ragged_b256_hq64_hkv8_d128_bs128_lognormal_k32",
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    chunk = 1 << 24
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_u.size, chunk):
        v = flat_u[s:s + chunk]
        r = ((v >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_o[s:s + chunk] = ((v + r) >> np.uint32(16)).astype(np.uint16)
    return out


@dataclass
class Workload:
    """One decode step's inputs. bf16 tensors are uint16 bit arrays."""
    config: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    context_lens: np.ndarray          # [B] int32
    block_tables: np.ndarray          # [B, max_blocks_per_seq] int32, unused = -1
    key_cache: np.ndarray             # [NB, bs, H_kv, D] uint16 (bf16 bits)
    value_cache: np.ndarray           # [NB, bs, H_kv, D] uint16
    query: np.ndarray                 # [B, H_q, D] uint16
    new_key: np.ndarray               # [T, H_kv, D] uint16 (T may be 0)
    new_value: np.ndarray             # [T, H_kv, D] uint16
    slot_mapping: np.ndarray          # [T] int64, <0 = skip
    topk_list: list = field(default_factory=list)   # Quest topk_blocks values to run
    scale: np.float32 = np.float32(0.0)
    # Multi-token queries (varlen): sequence b's query rows are
    # query_varlen[cu_seqlens_q[b]:cu_seqlens_q[b + 1]].
    cu_seqlens_q: np.ndarray | None = None  # [B + 1] int32
    query_varlen: np.ndarray | None = None  # [sum q_len, H_q, D] uint16

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def nblocks(self) -> np.ndarray:
        bs = self.block_size
        return (self.context_lens.astype(np.int64) + bs - 1) // bs


def _normal_bf16(rng: np.random.Generator, shape, offsets=None) -> np.ndarray:
    n = int(np.prod(shape))
    x = rng.standard_normal(n, dtype=np.float32).reshape(shape)
    if offsets is not None:
        offsets(x)
    return bf16_bits(x)


def _assign_blocks(rng, nb: np.ndarray, num_blocks: int, max_blocks: int) -> np.ndarray:
    """Physical ids = a random permutation of the pool, handed out in sequence order."""
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((nb.size, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nb):
        bt[b, :n] = perm[pos:pos + n]
        pos += int(n)
    return bt


def _slots_at_last_position(ctx, bt, bs, skip=None) -> np.ndarray:
    """The new token of sequence b is its last position ctx_b - 1."""
    pos = ctx.astype(np.int64) - 1
    lb = pos // bs
    slots = bt[np.arange(ctx.size), lb].astype(np.int64) * bs + pos % bs
    if skip is not None:
        slots[skip] = -1
    return slots


def make(config: int, seed: int | None = None) -> Workload:
    """Build workload 1..5 (see the module docstring) with ``seed`` (default: its number)."""
    if seed is None:
        seed = config
    rng = np.random.default_rng(seed)
    if config == 1:
        B, Hq, Hkv, D, bs, max_blocks, NB = 2, 4, 1, 64, 16, 5, 16
        ctx = np.array([37, 80], dtype=np.int32)
        nb = (ctx + bs - 1) // bs
        perm = rng.permutation(NB).astype(np.int32)
        bt = np.full((B, max_blocks), -1, dtype=np.int32)
        bt[0, :3] = perm[0:3]
        bt[1, :5] = perm[3:8]
        kc = _normal_bf16(rng, (NB, bs, Hkv, D))
        vc = _normal_bf16(rng, (NB, bs, Hkv, D))
        q = _normal_bf16(rng, (B, Hq, D))
        nk = _normal_bf16(rng, (2, Hkv, D))
        nv = _normal_bf16(rng, (2, Hkv, D))
        slots = np.array([_slots_at_last_position(ctx[:1], bt[:1], bs)[0], -1], dtype=np.int64)
        topk = [3, 5]
    elif config == 2:
        B, Hq, Hkv, D, bs, max_blocks = 32, 28, 4, 128, 128, 64
        ctx = rng.integers(1024, 8192, size=B, endpoint=True).astype(np.int32)
        nb = (ctx + bs - 1) // bs
        NB = int(math.ceil(1.1 * int(nb.sum())))
        bt = _assign_blocks(rng, nb, NB, max_blocks)
        kc = _normal_bf16(rng, (NB, bs, Hkv, D))
        vc = _normal_bf16(rng, (NB, bs, Hkv, D))
        q = _normal_bf16(rng, (B, Hq, D))
        nk = _normal_bf16(rng, (B, Hkv, D))
        nv = _normal_bf16(rng, (B, Hkv, D))
        slots = _slots_at_last_position(ctx, bt, bs)
        topk = []
    elif config == 3:
        B, Hq, Hkv, D, bs, max_blocks = 64, 28, 4, 128, 16, 1024
        ctx = np.clip(np.round(rng.normal(8192.0, 2048.0, size=B)), 2048, 16384).astype(np.int32)
        nb = (ctx + bs - 1) // bs
        NB = int(math.ceil(1.1 * int(nb.sum())))
        bt = _assign_blocks(rng, nb, NB, max_blocks)
        kc_f = rng.standard_normal(NB * bs * Hkv * D, dtype=np.float32).reshape(NB, bs, Hkv, D)
        vc = _normal_bf16(rng, (NB, bs, Hkv, D))
        q = _normal_bf16(rng, (B, Hq, D))
        nk = _normal_bf16(rng, (B, Hkv, D))
        nv = _normal_bf16(rng, (B, Hkv, D))
        slots = _slots_at_last_position(ctx, bt, bs)
        # Quest structure: 5% of (b, logical block, kv head) get +2.0 on 16 random
        # channels for every token of the block, before bf16 rounding.
        for b in range(B):
            for lb in range(int(nb[b])):
                hit = rng.random(Hkv) < 0.05
                for g in np.nonzero(hit)[0]:
                    ch = rng.choice(D, size=16, replace=False)
                    kc_f[bt[b, lb], :, g, ch] += np.float32(2.0)
        kc = bf16_bits(kc_f)
        del kc_f
        topk = [64]
    elif config == 4:
        B, Hq, Hkv, D, bs, max_blocks, NB = 4, 28, 4, 128, 16, 2560, 10240
        ctx = np.full(B, 40960, dtype=np.int32)
        nb = (ctx + bs - 1) // bs
        bt = _assign_blocks(rng, nb, NB, max_blocks)
        kc = _normal_bf16(rng, (NB, bs, Hkv, D))
        vc = _normal_bf16(rng, (NB, bs, Hkv, D))
        q = _normal_bf16(rng, (B, Hq, D))
        nk = np.zeros((0, Hkv, D), dtype=np.uint16)
        nv = np.zeros((0, Hkv, D), dtype=np.uint16)
        slots = np.zeros((0,), dtype=np.int64)
        topk = [256]
    elif config == 5:
        B, Hq, Hkv, D, bs, max_blocks = 256, 64, 8, 128, 128, 256
        ctx = np.clip(np.round(np.exp(rng.normal(math.log(1536.0), 1.0, size=B))), 1, 32768).astype(np.int32)
        nb = (ctx + bs - 1) // bs
        NB = int(math.ceil(1.1 * int(nb.sum())))
        bt = _assign_blocks(rng, nb, NB, max_blocks)
        kc = _normal_bf16(rng, (NB, bs, Hkv, D))
        vc = _normal_bf16(rng, (NB, bs, Hkv, D))
        q = _normal_bf16(rng, (B, Hq, D))
        nk = _normal_bf16(rng, (B, Hkv, D))
        nv = _normal_bf16(rng, (B, Hkv, D))
        skip = rng.choice(B, size=int(round(0.05 * B)), replace=False)
        slots = _slots_at_last_position(ctx, bt, bs, skip=skip)
        topk = [32]
    else:
        raise ValueError(f"unknown config {config}")
    return Workload(
        config=config, name=CONFIG_NAMES[config], batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=bs, num_blocks=int(kc.shape[0]), max_blocks_per_seq=max_blocks,
        context_lens=ctx, block_tables=bt, key_cache=kc, value_cache=vc, query=q,
        new_key=nk, new_value=nv, slot_mapping=slots, topk_list=topk,
        scale=np.float32(1.0 / math.sqrt(D)))


def random_case(seed: int, *, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, context_lens, max_blocks_per_seq: int | None = None,
                slack: int = 3, num_tokens: int = 0, neg_slots: int = 0) -> Workload:
    """A small free-shape case for parity tests (ragged tails, several tiles).

    ``context_lens`` may hold zeros. Physical blocks are a random permutation of a
    pool with ``slack`` spare blocks. New tokens (``num_tokens`` <= batch) sit at
    the last position of the first sequences with ctx > 0; ``neg_slots`` of them
    get slot -1.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int32)
    assert ctx.size == batch
    bs = block_size
    nb = (ctx.astype(np.int64) + bs - 1) // bs
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(nb.max()) if nb.size else 1)
    NB = int(nb.sum()) + slack
    bt = _assign_blocks(rng, nb, NB, max_blocks_per_seq)
    kc = _normal_bf16(rng, (NB, bs, num_kv_heads, head_dim))
    vc = _normal_bf16(rng, (NB, bs, num_kv_heads, head_dim))
    q = _normal_bf16(rng, (batch, num_q_heads, head_dim))
    live = np.nonzero(ctx > 0)[0][:num_tokens]
    T = live.size
    nk = _normal_bf16(rng, (T, num_kv_heads, head_dim))
    nv = _normal_bf16(rng, (T, num_kv_heads, head_dim))
    slots = _slots_at_last_position(ctx[live], bt[live], bs) if T else np.zeros((0,), np.int64)
    if neg_slots and T:
        slots[rng.choice(T, size=min(neg_slots, T), replace=False)] = -1
    return Workload(
        config=0, name=f"random_seed{seed}", batch=batch, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs, num_blocks=NB,
        max_blocks_per_seq=max_blocks_per_seq, context_lens=ctx, block_tables=bt,
        key_cache=kc, value_cache=vc, query=q, new_key=nk, new_value=nv, slot_mapping=slots,
        topk_list=[], scale=np.float32(1.0 / math.sqrt(head_dim)))


def varlen_case(seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, context_lens, q_lens, slack: int = 3) -> Workload:
    """Multi-token queries over a paged cache: sequence b brings q_lens[b] query
    tokens, the newest q_lens[b] of its context_lens[b] positions (their K/V already
    in the cache). Caches and tables as ``random_case(seed, ...)``; the query rows
    are drawn from a second seeded stream."""
    ctx = np.asarray(context_lens, dtype=np.int32)
    w = random_case(seed, batch=int(ctx.size), num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                    context_lens=ctx, slack=slack)
    ql = np.asarray(q_lens, dtype=np.int32)
    assert ql.size == ctx.size and (ql >= 0).all()
    cu = np.zeros(ctx.size + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    rng = np.random.default_rng(seed + 7919)
    w.query_varlen = _normal_bf16(rng, (int(cu[-1]), num_q_heads, head_dim))
    w.cu_seqlens_q = cu
    w.name = f"varlen_seed{seed}"
    return w


def shape_summary(w: Workload) -> dict:
    return {
        "workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
        "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
        "num_blocks": w.num_blocks, "max_blocks_per_seq": w.max_blocks_per_seq,
        "sum_context": int(w.context_lens.sum()), "max_context_len": w.max_context_len,
        "new_tokens": w.num_tokens, "topk_blocks": list(w.topk_list),
    }
