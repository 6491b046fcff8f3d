"""Helpers shared by the GPU tests: upload a workload, download results."""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import workloads

BF = torch.bfloat16


def to_dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == BF:
        return torch.from_numpy(a.view(np.int16)).view(BF).cuda()
    return torch.from_numpy(a).to(dtype).cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class Dev:
    """A workload's tensors on cuda:0."""

    def __init__(self, w: workloads.Workload):
        self.w = w
        self.kc = to_dev(w.key_cache, BF)
        self.vc = to_dev(w.value_cache, BF)
        self.q = to_dev(w.query, BF)
        self.bt = to_dev(w.block_tables, torch.int32)
        self.ctx = to_dev(w.context_lens, torch.int32)
        self.nk = to_dev(w.new_key, BF)
        self.nv = to_dev(w.new_value, BF)
        self.slots = to_dev(w.slot_mapping, torch.int64)


@functools.lru_cache(maxsize=None)
def workload(config: int) -> workloads.Workload:
    return workloads.make(config)


# ---------------------------------------------------------------------------
# Oracle results over every sequence of a full-size workload, computed once per
# test session (several tests and schedules compare against the same result).
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def step_caches(config: int):
    """(key_cache, value_cache) bits after the step's write, by the oracle."""
    w = workload(config)
    if not w.num_tokens:
        return w.key_cache, w.value_cache
    return oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                    w.slot_mapping, w.block_size)


@functools.lru_cache(maxsize=None)
def dense_ref(config: int) -> np.ndarray:
    """Dense attention of every sequence over the caches after the step's write."""
    w = workload(config)
    kc, vc = step_caches(config)
    return oracle.paged_attention_decode(w.query, kc, vc, w.block_tables, w.context_lens,
                                         w.scale)


@functools.lru_cache(maxsize=None)
def oracle_selection(config: int, K: int) -> np.ndarray:
    """Top-K of every (sequence, KV head) from metadata over the generated pool."""
    w = workload(config)
    omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens,
                                             w.block_size)
    return oracle.quest_select_topk(w.query, omin, omax, w.block_tables, w.context_lens,
                                    w.block_size, K)


@functools.lru_cache(maxsize=None)
def sparse_ref(config: int, K: int) -> np.ndarray:
    """Sparse attention of every sequence over the generated pool, the selection
    fixed to the oracle's Top-K."""
    w = workload(config)
    return oracle.sparse_paged_attention_decode(w.query, w.key_cache, w.value_cache,
                                                w.block_tables, w.context_lens,
                                                oracle_selection(config, K), w.scale)


def fp8_codes(cache_bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The oracle's E4M3 codes of a whole bf16 cache [..., H_kv, D]. quantize_fp8 is an
    elementwise function of (bf16 pattern, KV head), so it is evaluated once on all
    65536 patterns for each head and then looked up: the same codes as calling it on
    the cache, in seconds rather than minutes at full size."""
    Hkv = cache_bits.shape[-2]
    allbits = np.repeat(np.arange(65536, dtype=np.uint16)[:, None, None], Hkv, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):   # the table spans inf and NaN patterns
        table = oracle.quantize_fp8(allbits, scales)[:, :, 0]      # [65536, H_kv]
    out = np.empty(cache_bits.shape, np.uint8)
    for g in range(Hkv):
        out[..., g, :] = table[:, g][cache_bits[..., g, :]]
    return out


def sample_seqs(w: workloads.Workload, n: int = 6, seed: int = 0) -> list[int]:
    """Longest, shortest and a few seeded random sequences (oracle cost stays small)."""
    ctx = w.context_lens
    rng = np.random.default_rng(1000 + seed)
    pick = {int(np.argmax(ctx)), int(np.argmin(ctx))}
    extra = rng.choice(w.batch, size=min(w.batch, n), replace=False)
    for b in extra.tolist():
        if len(pick) >= n:
            break
        pick.add(int(b))
    return sorted(pick)


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)).max())


# ---------------------------------------------------------------------------
# The write path: metadata comparisons and the pre-write context
# ---------------------------------------------------------------------------

SENTINEL = 0x1234   # fills metadata rows no call should touch


def meta_equal(got, exp) -> bool:
    """Bitwise, except +0 and -0 count as equal."""
    g = got.copy()
    e = exp.copy()
    g[g == 0x8000] = 0
    e[e == 0x8000] = 0
    return np.array_equal(g, e)


def before_write_lens(w: workloads.Workload) -> np.ndarray:
    """Context lengths before this step's write: ctx - 1 for a sequence whose
    newest slot (position ctx - 1) is written by a valid slot of slot_mapping."""
    ctx, bt, bs = w.context_lens.astype(np.int64), w.block_tables, w.block_size
    valid = set(int(s) for s in w.slot_mapping if 0 <= s < w.num_blocks * bs)
    before = ctx.copy()
    for b in np.nonzero(ctx > 0)[0]:
        pos = ctx[b] - 1
        if int(bt[b, pos // bs]) * bs + int(pos % bs) in valid:
            before[b] -= 1
    return before.astype(np.int32)
