"""The dense decode call with the step's cache write (decode append) against the
oracle chain: ReshapeAndCache (and the Quest key min / max fold) over the batch's
new tokens, then dense attention over the written caches.

Source: "Ascend Kernel-to-Serving Pipeline", sections "ReshapeAndCache" and "GQA
Paged Attention"; the per-step write merged into the decode launch is the sparse-
attention adaptation article's item 3 of its four key levels. Caches and metadata
must match bit for bit, attention within 2e-3 (the bf16-input, fp32-accumulation
bar), on every sequence."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import (BF, SENTINEL, Dev, before_write_lens, bits, dense_ref, max_abs, meta_equal,
                      step_caches, to_dev, workload)

pytestmark = pytest.mark.gpu
ATOL = 2e-3
SCHEDULES = ["balanced", "split"]


def _append(d, w, kmin=None, kmax=None, workspace=None):
    return gp.paged_attention_decode_append(
        d.q, d.nk, d.nv, d.kc, d.vc, d.slots, d.bt, d.ctx, max_context_len=w.max_context_len,
        scale=float(w.scale), key_min=kmin, key_max=kmax, workspace=workspace)


def _one_token_per_sequence(w):
    assert w.num_tokens == w.batch, "decode append writes token b for sequence b"


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("config", [1, 2, 5])
def test_append_config(config, schedule, monkeypatch):
    """Full-size workloads with a write: every sequence's output and both whole caches."""
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workload(config)
    _one_token_per_sequence(w)
    d = Dev(w)
    out = _append(d, w)
    torch.cuda.synchronize()
    ek, ev = step_caches(config)
    assert np.array_equal(bits(d.kc), ek), "key cache differs from the oracle"
    assert np.array_equal(bits(d.vc), ev), "value cache differs from the oracle"
    err = max_abs(out.cpu().numpy(), dense_ref(config))
    assert err <= ATOL, f"config {config}: max abs error {err}"


def _check_random(w, schedule, monkeypatch, with_meta):
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    _one_token_per_sequence(w)
    d = Dev(w)
    kmin = kmax = None
    if with_meta:
        # metadata over the pre-write contexts, the decode-append starting point
        base = np.full((w.num_blocks, w.num_kv_heads, w.head_dim), SENTINEL, np.uint16)
        pmin, pmax = oracle.quest_block_metadata(w.key_cache, w.block_tables, before_write_lens(w),
                                                 w.block_size, last_block_only=True,
                                                 key_min=base, key_max=base)
        kmin, kmax = to_dev(pmin, BF), to_dev(pmax, BF)
    out = _append(d, w, kmin, kmax)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                      w.slot_mapping, w.block_size)
    assert np.array_equal(bits(d.kc), ek), "key cache differs from the oracle"
    assert np.array_equal(bits(d.vc), ev), "value cache differs from the oracle"
    ref = oracle.paged_attention_decode(w.query, ek, ev, w.block_tables, w.context_lens, w.scale)
    err = max_abs(out.cpu().numpy(), ref)
    assert err <= ATOL, f"max abs error {err}"
    if with_meta:
        emin, emax = oracle.quest_block_metadata(ek, w.block_tables, w.context_lens, w.block_size,
                                                 last_block_only=True, key_min=pmin, key_max=pmax)
        assert meta_equal(bits(kmin), emin), "key_min differs from the oracle chain"
        assert meta_equal(bits(kmax), emax), "key_max differs from the oracle chain"
    return out


# Contexts put the new token at row 0 of a block, at its last row and in between; a
# context of 1 leaves the new token alone; long contexts give many units per
# sequence (the per-query-head combine), short batches few (the per-KV-head one).
RANDOM = [
    (601, 8, 1, 64, 16, [1, 2, 16, 17, 33, 64, 65, 100], 2),
    (602, 28, 4, 128, 16, [1, 5000, 17, 2049, 300], 1),
    (603, 64, 8, 128, 128, [129, 128, 1, 700, 1536, 4097], 2),
    (604, 16, 2, 64, 64, [64, 65, 3000], 0),
    (605, 32, 4, 128, 32, [31, 32, 33, 9000], 1),
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx,neg", RANDOM)
def test_append_random(seed, Hq, Hkv, D, bs, ctx, neg, schedule, monkeypatch):
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=ctx, num_tokens=len(ctx), neg_slots=neg)
    _check_random(w, schedule, monkeypatch, with_meta=True)


def test_append_many_sequences_per_kv_head_combine(monkeypatch):
    """A batch large enough that the combine takes one workgroup per KV head."""
    rng = np.random.default_rng(606)
    ctx = rng.integers(1, 700, size=96).tolist()
    w = workloads.random_case(606, batch=96, num_q_heads=16, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=ctx, num_tokens=96, neg_slots=5)
    _check_random(w, "balanced", monkeypatch, with_meta=False)


def test_append_single_token_context_is_the_new_value(monkeypatch):
    """With context 1 the softmax holds the new token alone: the output is its value."""
    w = workloads.random_case(607, batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[1, 1, 1], num_tokens=3)
    out = _check_random(w, "balanced", monkeypatch, with_meta=False).cpu().numpy()
    v = oracle.bf16_to_f64(w.new_value)          # [B, H_kv, D]
    exp = np.repeat(v, 4, axis=1)                # query head h reads KV head h / 4
    assert np.array_equal(out.astype(np.float64), exp)


def test_append_empty_context_still_writes(monkeypatch):
    """A sequence of context 0 whose token has a slot: the token is written (as
    ReshapeAndCache writes it) and the sequence's output row is zero."""
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", "balanced")
    w = workloads.random_case(608, batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
                              block_size=16, context_lens=[0, 40], num_tokens=0, slack=2)
    rng = np.random.default_rng(608)
    used = set(int(x) for x in w.block_tables[w.block_tables >= 0].ravel())
    free = [pb for pb in range(w.num_blocks) if pb not in used][0]
    pos = 39
    slots = np.array([free * 16 + 5, int(w.block_tables[1, pos // 16]) * 16 + pos % 16], np.int64)
    nk = workloads.bf16_bits(rng.standard_normal((2, 1, 64), dtype=np.float32))
    nv = workloads.bf16_bits(rng.standard_normal((2, 1, 64), dtype=np.float32))
    d = Dev(w)
    d.nk, d.nv, d.slots = to_dev(nk, BF), to_dev(nv, BF), to_dev(slots, torch.int64)
    out = gp.paged_attention_decode_append(d.q, d.nk, d.nv, d.kc, d.vc, d.slots, d.bt, d.ctx,
                                           max_context_len=40, scale=float(w.scale))
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(w.key_cache, w.value_cache, nk, nv, slots, 16)
    assert np.array_equal(bits(d.kc), ek) and np.array_equal(bits(d.vc), ev)
    ref = oracle.paged_attention_decode(w.query, ek, ev, w.block_tables, w.context_lens, w.scale)
    o = out.cpu().numpy()
    assert np.all(o[0] == 0.0)
    assert max_abs(o, ref) <= ATOL


def test_append_equals_write_then_decode_on_the_gpu(monkeypatch):
    """The same step as two calls on the GPU (write, then dense decode): caches equal
    bit for bit, outputs within the bar (the appended token is merged as its own
    unit, so the float32 sums are grouped differently)."""
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", "balanced")
    w = workload(5)
    a, b = Dev(w), Dev(w)
    out_a = _append(a, w)
    gp.reshape_and_cache(b.nk, b.nv, b.kc, b.vc, b.slots)
    out_b = gp.paged_attention_decode(b.q, b.kc, b.vc, b.bt, b.ctx,
                                      max_context_len=w.max_context_len, scale=float(w.scale))
    torch.cuda.synchronize()
    assert torch.equal(a.kc, b.kc) and torch.equal(a.vc, b.vc)
    assert float((out_a - out_b).abs().max()) <= 1e-4


def _spiked(seed, ctx, D=128, H=4, bs=16):
    """One query head per KV head and each new key along its head's query, sized so that
    the new token's score is the log of the other tokens' summed weight: it carries
    about half of its sequence's softmax, so a slip in its unit (left out, its scale,
    its lse, its values) moves the output by O(0.1)."""
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=H, num_kv_heads=H, head_dim=D,
                              block_size=bs, context_lens=ctx, num_tokens=len(ctx))
    w.new_key[...] = spike_keys(w)
    return w


def spike_keys(w):
    """k_new[b, h] = a q[b, h] with a chosen so that scale * q . k_new equals
    ln(sum over the other tokens of exp(score)), about ln(ctx - 1) + 1/2 for random
    keys (their scores are close to standard normal)."""
    q = oracle.bf16_to_f64(w.query)                       # [B, H, D]
    s = float(w.scale)
    target = np.log(np.maximum(w.context_lens.astype(np.float64) - 1, 1)) + 0.5
    a = target[:, None] / (s * (q * q).sum(axis=-1))      # [B, H]
    return workloads.bf16_bits((a[..., None] * q).astype(np.float32))


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_append_spiked_new_token(schedule, monkeypatch):
    w = _spiked(611, [9000, 3000, 2])
    _check_random(w, schedule, monkeypatch, with_meta=True)
