"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Bars: cache writes, Quest metadata and Top-K indices bit-exact; attention outputs
within max-abs 2e-3 of the float64 oracle (bf16 inputs, fp32 accumulation).
Full-size configs compare every output -- caches, metadata, indices and the
attention rows of every sequence -- in the launch configuration the benchmark
uses.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import (BF, SENTINEL, Dev, bits, dense_ref, max_abs, oracle_selection, sparse_ref,
                      to_dev, workload)
from gpu_util import before_write_lens as _before_write_lens
from gpu_util import meta_equal as _meta_equal

pytestmark = pytest.mark.gpu
ATOL = 2e-3


# ---------------------------------------------------------------------------
# ReshapeAndCache
# ---------------------------------------------------------------------------

def _check_write(w):
    d = Dev(w)
    gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, d.slots)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                      w.slot_mapping, w.block_size)
    assert np.array_equal(bits(d.kc), ek), "key cache differs from the oracle"
    assert np.array_equal(bits(d.vc), ev), "value cache differs from the oracle"
    return d


@pytest.mark.parametrize("config", [1, 2, 3, 5])
def test_reshape_and_cache_config(config):
    _check_write(workload(config))


@pytest.mark.parametrize("seed,Hkv,D,bs", [(101, 1, 64, 16), (102, 4, 128, 32), (103, 8, 128, 128),
                                           (104, 2, 64, 64)])
def test_reshape_and_cache_random(seed, Hkv, D, bs):
    w = workloads.random_case(seed, batch=9, num_q_heads=Hkv * 2, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=[1, 5, 16, 17, 40, 64, 100, 129, 300],
                              num_tokens=9, neg_slots=3)
    _check_write(w)


def test_reshape_and_cache_all_negative_and_empty():
    w = workloads.make(1)
    d = Dev(w)
    before_k, before_v = bits(d.kc), bits(d.vc)
    gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, torch.full_like(d.slots, -1))
    empty_k = torch.empty((0, 1, 64), dtype=BF, device="cuda")
    gp.reshape_and_cache(empty_k, empty_k, d.kc, d.vc, torch.empty((0,), dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(bits(d.kc), before_k) and np.array_equal(bits(d.vc), before_v)


# ---------------------------------------------------------------------------
# Dense attention
# ---------------------------------------------------------------------------

def _dense(d, w, **kw):
    return gp.paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx, max_context_len=w.max_context_len,
                                     scale=float(w.scale), **kw)


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_dense_config(config):
    w = workload(config)
    d = Dev(w)
    if w.num_tokens:   # the step writes the new token first (context_lens include it)
        gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, d.slots)
    out = _dense(d, w).cpu().numpy()
    err = max_abs(out, dense_ref(config))
    print(f"config {config}: dense max-abs {err:.3e} over all {w.batch} sequences")
    assert err <= ATOL
    assert np.isfinite(out).all()


DENSE_CASES = [
    # seed, Hq, Hkv, D, bs, context lengths
    (201, 4, 1, 64, 16, [0, 1, 15, 16, 17, 33]),
    (202, 28, 4, 128, 16, [31, 32, 33, 500, 1023, 1025]),
    (203, 16, 16, 128, 32, [7, 64, 65, 300]),             # G = 1 (MHA)
    (204, 16, 1, 128, 64, [129, 2047, 4100]),              # G = 16 (largest group)
    (205, 64, 8, 128, 128, [1, 127, 128, 129, 3000, 5000]),
    (206, 14, 2, 64, 128, [250, 1, 700]),
    (207, 12, 3, 64, 32, [513, 514, 96]),
]


SCHEDULES = ["balanced", "split"]
# Sparse calls also have the direct path (one workgroup per sequence and KV head),
# the default when those pairs fill the GPU; forcing it covers small batches too.
SPARSE_SCHEDULES = SCHEDULES + ["direct"]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx", DENSE_CASES)
def test_dense_random(seed, Hq, Hkv, D, bs, ctx, schedule, monkeypatch):
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=ctx)
    d = Dev(w)
    out = _dense(d, w).cpu().numpy()
    ref = oracle.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                        w.context_lens, w.scale)
    err = max_abs(out, ref)
    print(f"seed {seed}: max-abs {err:.3e}")
    assert err <= ATOL
    for b, L in enumerate(ctx):
        if L == 0:
            assert (out[b] == 0).all(), "empty context -> zero row"


@pytest.mark.parametrize("split", [128, 256, 512, 1024, 2048])
def test_dense_split_sizes_agree(split, monkeypatch):
    """Any split partition gives the same attention (the combine identity)."""
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", "split")
    monkeypatch.setenv("GPKV_SPLIT_TOKENS", str(split))
    assert gp.split_tokens(3, 4, 4000) == split
    w = workloads.random_case(210, batch=3, num_q_heads=28, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=[4000, 2500, 129])
    d = Dev(w)
    ref = oracle.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                        w.context_lens, w.scale)
    out = _dense(d, w).cpu().numpy()
    assert max_abs(out, ref) <= ATOL
    sel = np.full((3, 4, 250), -1, np.int32)
    for b, nb in enumerate(w.nblocks().tolist()):
        sel[b, :, :nb] = np.arange(nb)
    sp = _sparse(d, w, to_dev(sel, torch.int32)).cpu().numpy()
    assert max_abs(sp, ref) <= ATOL


def test_balanced_workspace_reused_across_batches():
    """One workspace through calls of different batches, dense then sparse: the
    arrival counters return to zero after every call, so each call merges."""
    cases = [workloads.random_case(215 + i, batch=len(ctx), num_q_heads=28, num_kv_heads=4,
                                   head_dim=128, block_size=16, context_lens=ctx)
             for i, ctx in enumerate([[900, 0, 2500, 16], [3000, 1], [17, 400, 0, 5000, 33, 1]])]
    need = max(gp.paged_attention_workspace_bytes(w.batch, 28, 4, 128, 16, w.max_context_len)
               for w in cases)
    need = max(need, max(gp.sparse_attention_workspace_bytes(w.batch, 28, 4, 128, 16, 400)
                         for w in cases))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for w in cases:
            d = Dev(w)
            out = torch.full((w.batch, 28, 128), float("nan"), device="cuda")
            _dense(d, w, out=out, workspace=ws)
            ref = oracle.paged_attention_decode(w.query, w.key_cache, w.value_cache,
                                                w.block_tables, w.context_lens, w.scale)
            assert max_abs(out.cpu().numpy(), ref) <= ATOL, (rep, w.batch)
            sel = np.full((w.batch, 4, 400), -1, np.int32)
            for b, nb in enumerate(w.nblocks().tolist()):
                sel[b, :, :nb] = np.arange(nb)
            sp = torch.full((w.batch, 28, 128), float("nan"), device="cuda")
            gp.sparse_paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx, to_dev(sel, torch.int32),
                                             max_context_len=w.max_context_len,
                                             scale=float(w.scale), out=sp, workspace=ws)
            assert max_abs(sp.cpu().numpy(), ref) <= ATOL, (rep, w.batch)


def test_dense_invariants_permuted_poison_deterministic():
    w = workloads.random_case(220, batch=4, num_q_heads=28, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=[700, 37, 1600, 16], slack=9)
    d = Dev(w)
    out1 = _dense(d, w)
    out2 = _dense(d, w)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "two runs differ bitwise"
    # NaN in every row outside the contexts (incl. unreferenced blocks) changes nothing.
    kc = w.key_cache.copy()
    vc = w.value_cache.copy()
    live = np.zeros(kc.shape[:2], dtype=bool)
    for b in range(w.batch):
        for t in range(int(w.context_lens[b])):
            live[int(w.block_tables[b, t // 16]), t % 16] = True
    kc[~live] = 0x7FC0
    vc[~live] = 0x7FC0
    d2 = Dev(w)
    d2.kc, d2.vc = to_dev(kc, BF), to_dev(vc, BF)
    out3 = _dense(d2, w)
    torch.cuda.synchronize()
    assert torch.equal(out1, out3), "NaN outside the context leaked into the output"
    # Moving every physical block (data copied along) leaves the output unchanged.
    perm = np.random.default_rng(7).permutation(w.num_blocks)
    kp = np.empty_like(w.key_cache)
    vp = np.empty_like(w.value_cache)
    kp[perm] = w.key_cache
    vp[perm] = w.value_cache
    btp = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    d3 = Dev(w)
    d3.kc, d3.vc, d3.bt = to_dev(kp, BF), to_dev(vp, BF), to_dev(btp, torch.int32)
    out4 = _dense(d3, w)
    torch.cuda.synchronize()
    assert torch.equal(out1, out4), "permuted block table changed the output"


# ---------------------------------------------------------------------------
# Quest metadata, Top-K, sparse attention
# ---------------------------------------------------------------------------

def _meta(d, w, last_only=False, kmin=None, kmax=None):
    if kmin is None:
        kmin = to_dev(np.full((w.num_blocks, w.num_kv_heads, w.head_dim), SENTINEL, np.uint16), BF)
        kmax = to_dev(np.full((w.num_blocks, w.num_kv_heads, w.head_dim), SENTINEL, np.uint16), BF)
    gp.quest_block_metadata(d.kc, d.bt, d.ctx, kmin, kmax, max_context_len=w.max_context_len,
                            last_block_only=last_only)
    return kmin, kmax


@pytest.mark.parametrize("config", [1, 3, 4, 5])
def test_quest_metadata_config(config):
    w = workload(config)
    d = Dev(w)
    kmin, kmax = _meta(d, w)
    torch.cuda.synchronize()
    base = np.full((w.num_blocks, w.num_kv_heads, w.head_dim), SENTINEL, np.uint16)
    emin, emax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens,
                                             w.block_size, key_min=base, key_max=base)
    assert _meta_equal(bits(kmin), emin) and _meta_equal(bits(kmax), emax)


def test_quest_metadata_step_after_write():
    """Write the new tokens, refresh only each sequence's last block."""
    w = workloads.random_case(301, batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128,
                              block_size=16, context_lens=[1, 16, 17, 100, 250, 33],
                              num_tokens=6, neg_slots=1)
    d = Dev(w)
    base = np.full((w.num_blocks, w.num_kv_heads, w.head_dim), SENTINEL, np.uint16)
    kmin, kmax = to_dev(base, BF), to_dev(base, BF)
    gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, d.slots)
    _meta(d, w, last_only=True, kmin=kmin, kmax=kmax)
    torch.cuda.synchronize()
    kc, _ = oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                     w.slot_mapping, w.block_size)
    emin, emax = oracle.quest_block_metadata(kc, w.block_tables, w.context_lens, w.block_size,
                                             last_block_only=True, key_min=base, key_max=base)
    assert _meta_equal(bits(kmin), emin) and _meta_equal(bits(kmax), emax)


def _check_fused_write(w):
    """reshape_and_cache_quest against the oracle chain: write, then refresh each
    sequence's last block, starting from metadata that covers the pre-write
    context (the decode-append contract)."""
    before = _before_write_lens(w)
    assert (before < w.context_lens).any(), "the case writes no token"
    base = np.full((w.num_blocks, w.num_kv_heads, w.head_dim), SENTINEL, np.uint16)
    pmin, pmax = oracle.quest_block_metadata(w.key_cache, w.block_tables, before, w.block_size,
                                             last_block_only=True, key_min=base, key_max=base)
    d = Dev(w)
    kmin, kmax = to_dev(pmin, BF), to_dev(pmax, BF)
    gp.reshape_and_cache_quest(d.nk, d.nv, d.kc, d.vc, kmin, kmax, d.slots)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                      w.slot_mapping, w.block_size)
    assert np.array_equal(bits(d.kc), ek), "key cache differs from the oracle"
    assert np.array_equal(bits(d.vc), ev), "value cache differs from the oracle"
    emin, emax = oracle.quest_block_metadata(ek, w.block_tables, w.context_lens, w.block_size,
                                             last_block_only=True, key_min=pmin, key_max=pmax)
    assert _meta_equal(bits(kmin), emin), "key_min differs from the oracle chain"
    assert _meta_equal(bits(kmax), emax), "key_max differs from the oracle chain"


@pytest.mark.parametrize("config", [1, 3, 5])
def test_fused_write_config(config):
    _check_fused_write(workload(config))


@pytest.mark.parametrize("seed,Hkv,D,bs", [(501, 1, 64, 16), (502, 4, 128, 16), (503, 8, 128, 128),
                                           (504, 2, 64, 64), (505, 4, 128, 32)])
def test_fused_write_random(seed, Hkv, D, bs):
    """Context lengths put the new token at row 0, at the last row, and in between."""
    ctx = [1, 2, 16, 17, 33, 64, 65, 100, 128, 129, 257, 300]
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hkv * 2, num_kv_heads=Hkv,
                              head_dim=D, block_size=bs, context_lens=ctx, num_tokens=len(ctx),
                              neg_slots=2)
    _check_fused_write(w)


def test_fused_write_empty_and_all_negative():
    w = workloads.make(1)
    d = Dev(w)
    kmin = to_dev(np.full((w.num_blocks, 1, 64), SENTINEL, np.uint16), BF)
    kmax = kmin.clone()
    before = [bits(t) for t in (d.kc, d.vc, kmin, kmax)]
    gp.reshape_and_cache_quest(d.nk, d.nv, d.kc, d.vc, kmin, kmax, torch.full_like(d.slots, -1))
    empty = torch.empty((0, 1, 64), dtype=BF, device="cuda")
    gp.reshape_and_cache_quest(empty, empty, d.kc, d.vc, kmin, kmax,
                               torch.empty((0,), dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    for a, t in zip(before, (d.kc, d.vc, kmin, kmax)):
        assert np.array_equal(bits(t), a)


def test_fused_write_then_quest_step_matches_oracle_chain():
    """Full build at prefill, fused write at decode, then select + sparse."""
    w = workloads.random_case(341, batch=5, num_q_heads=28, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=[2000, 700, 17, 1234, 3001],
                              num_tokens=5, neg_slots=1)
    K = 24
    before = _before_write_lens(w)
    d = Dev(w)
    base = np.zeros((w.num_blocks, 4, 128), np.uint16)
    kmin, kmax = to_dev(base, BF), to_dev(base, BF)
    d_ctx_before = to_dev(before, torch.int32)
    gp.quest_block_metadata(d.kc, d.bt, d_ctx_before, kmin, kmax,
                            max_context_len=w.max_context_len)       # prefill-time build
    gp.reshape_and_cache_quest(d.nk, d.nv, d.kc, d.vc, kmin, kmax, d.slots)
    sel = gp.quest_select_topk(d.q, kmin, kmax, d.bt, d.ctx, block_size=16, topk_blocks=K,
                               max_context_len=w.max_context_len)
    out = _sparse(d, w, sel)
    torch.cuda.synchronize()
    kc, vc = oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                      w.slot_mapping, 16)
    omin, omax = oracle.quest_block_metadata(kc, w.block_tables, w.context_lens, 16,
                                             key_min=base, key_max=base)
    osel = oracle.quest_select_topk(w.query, omin, omax, w.block_tables, w.context_lens, 16, K)
    assert np.array_equal(sel.cpu().numpy(), osel)
    ref = oracle.sparse_paged_attention_decode(w.query, kc, vc, w.block_tables, w.context_lens,
                                               osel, w.scale)
    assert max_abs(out.cpu().numpy(), ref) <= ATOL


def _topk_case(w, K):
    d = Dev(w)
    kmin, kmax = _meta(d, w)
    sel = gp.quest_select_topk(d.q, kmin, kmax, d.bt, d.ctx, block_size=w.block_size,
                               topk_blocks=K, max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, w.block_size)
    exp = oracle.quest_select_topk(w.query, omin, omax, w.block_tables, w.context_lens,
                                   w.block_size, K)
    return d, sel.cpu().numpy(), exp


@pytest.mark.parametrize("path", ["auto", "fused", "two_kernel"])
@pytest.mark.parametrize("config,K", [(1, 3), (1, 5), (3, 64), (4, 256), (5, 32)])
def test_quest_topk_config(config, K, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("GPKV_QUEST_SELECT_PATH", path)
    w = workload(config)
    _, got, exp = _topk_case(w, K)
    mism = int((got != exp).any(axis=2).sum())
    assert mism == 0, f"{mism} (b, g) rows differ from the oracle"


@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx,K", [
    (311, 8, 2, 64, 16, [1, 100, 16, 1000, 4000], 7),
    (312, 28, 4, 128, 32, [2000, 33, 640], 1),
    (313, 64, 8, 128, 128, [129, 9000, 256], 5),
    (314, 16, 16, 128, 64, [3000], 40),
])
def test_quest_topk_random(seed, Hq, Hkv, D, bs, ctx, K):
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=ctx)
    _, got, exp = _topk_case(w, K)
    assert np.array_equal(got, exp)


def test_quest_topk_tie_goes_to_lower_block():
    w = workloads.random_case(320, batch=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                              block_size=16, context_lens=[640])
    omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    s = oracle.quest_block_scores(w.query, omin, omax, w.block_tables, w.context_lens, 16, 0, 0)
    order = np.argsort(-s, kind="stable")
    a = int(order[0])
    later = max(lb for lb in range(40) if lb != a)
    kc = w.key_cache.copy()
    kc[int(w.block_tables[0, later])] = kc[int(w.block_tables[0, a])]
    w.key_cache = kc
    for K in (1, 2, 3):
        _, got, exp = _topk_case(w, K)
        assert np.array_equal(got, exp), K
        assert min(a, later) in got[0, 0].tolist()


def _sparse(d, w, sel):
    return gp.sparse_paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx, sel,
                                            max_context_len=w.max_context_len,
                                            scale=float(w.scale))


@pytest.mark.parametrize("schedule", SPARSE_SCHEDULES)
@pytest.mark.parametrize("config,K", [(1, 3), (1, 5), (3, 64), (4, 256), (5, 32)])
def test_sparse_config_fixed_selection(config, K, schedule, monkeypatch):
    """Sparse kernel judged with the selection fixed to the oracle's Top-K."""
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workload(config)
    d = Dev(w)
    sel = oracle_selection(config, K)
    out = _sparse(d, w, to_dev(sel, torch.int32)).cpu().numpy()
    err = max_abs(out, sparse_ref(config, K))
    print(f"config {config} K={K}: sparse max-abs {err:.3e} over all {w.batch} sequences")
    assert err <= ATOL


@pytest.mark.parametrize("schedule", SPARSE_SCHEDULES)
def test_sparse_all_blocks_equals_dense_and_handles_holes(schedule, monkeypatch):
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workloads.random_case(330, batch=3, num_q_heads=28, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=[300, 17, 1000])
    d = Dev(w)
    nb = w.nblocks()
    K = int(nb.max()) + 3
    sel = np.full((3, 4, K), -1, np.int32)
    for b in range(3):
        sel[b, :, :nb[b]] = np.arange(nb[b])
    dense = _dense(d, w).cpu().numpy()
    sp = _sparse(d, w, to_dev(sel, torch.int32)).cpu().numpy()
    ref = oracle.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                        w.context_lens, w.scale)
    assert max_abs(sp, ref) <= ATOL and max_abs(dense, ref) <= ATOL
    # -1 holes and unsorted ids in the middle of the list, per KV head.
    sel2 = np.full((3, 4, 6), -1, np.int32)
    sel2[0, 0] = [5, -1, 2, 18, -1, 0]
    sel2[0, 1] = [-1, -1, -1, -1, -1, 1]
    sel2[1, 2] = [1, 0, -1, -1, -1, -1]
    sel2[1, 3] = [-1, -1, -1, -1, 1, 0]   # valid ids only past position min(K, blocks) = 2
    sel2[2, 3] = [62, 61, 3, -1, 9, 10]
    out = _sparse(d, w, to_dev(sel2, torch.int32)).cpu().numpy()
    ref2 = oracle.sparse_paged_attention_decode(w.query, w.key_cache, w.value_cache,
                                                w.block_tables, w.context_lens, sel2, w.scale)
    assert max_abs(out, ref2) <= ATOL
    assert (out[1, :8] == 0).all(), "no block selected -> zero rows"


# ---------------------------------------------------------------------------
# Composed Quest step, one stage swapped at a time
# ---------------------------------------------------------------------------

def test_composed_quest_step_matches_oracle_chain():
    w = workloads.random_case(340, batch=5, num_q_heads=28, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=[2000, 700, 16, 1234, 3001],
                              num_tokens=5, neg_slots=1)
    K = 24
    d = Dev(w)
    base = np.zeros((w.num_blocks, 4, 128), np.uint16)
    kmin, kmax = to_dev(base, BF), to_dev(base, BF)
    _meta(d, w, kmin=kmin, kmax=kmax)                       # prefill-time full build
    gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, d.slots)  # decode step: write
    _meta(d, w, last_only=True, kmin=kmin, kmax=kmax)      # refresh the last blocks
    sel = gp.quest_select_topk(d.q, kmin, kmax, d.bt, d.ctx, block_size=16, topk_blocks=K,
                               max_context_len=w.max_context_len)
    out = _sparse(d, w, sel)
    torch.cuda.synchronize()
    kc, vc = oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                      w.slot_mapping, 16)
    omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16,
                                             key_min=base, key_max=base)
    omin, omax = oracle.quest_block_metadata(kc, w.block_tables, w.context_lens, 16,
                                             last_block_only=True, key_min=omin, key_max=omax)
    osel = oracle.quest_select_topk(w.query, omin, omax, w.block_tables, w.context_lens, 16, K)
    assert np.array_equal(sel.cpu().numpy(), osel)
    ref = oracle.sparse_paged_attention_decode(w.query, kc, vc, w.block_tables, w.context_lens,
                                               osel, w.scale)
    assert max_abs(out.cpu().numpy(), ref) <= ATOL


def test_quest_topk_fused_path_ties_and_ragged():
    """Enough (sequence, KV head) pairs for the one-launch select path: ragged lengths,
    K above and below nb, and an exact tie planted in two sequences."""
    rng = np.random.default_rng(350)
    ctx = rng.integers(1, 9000, size=32).tolist()
    ctx[3], ctx[7], ctx[9] = 480, 640, 8500      # one table of more than 512 blocks
    w = workloads.random_case(350, batch=32, num_q_heads=28, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=ctx)
    kc = w.key_cache.copy()
    for b in (3, 7):   # copy the best block of KV head 0 into a later block of the sequence
        omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
        s = oracle.quest_block_scores(w.query, omin, omax, w.block_tables, w.context_lens, 16, b, 0)
        a = int(np.argmax(s))
        later = int(s.size - 1 if a != s.size - 1 else s.size - 2)
        kc[int(w.block_tables[b, later])] = kc[int(w.block_tables[b, a])]
    w.key_cache = kc
    for K in (1, 5, 24, 300):
        _, got, exp = _topk_case(w, K)
        assert np.array_equal(got, exp), K


@pytest.mark.parametrize("ctx,Hkv", [([110000], 2), ([9000, 700, 20000], 1)])
def test_quest_topk_few_pairs_long_tables(ctx, Hkv, monkeypatch):
    """Few (sequence, KV head) pairs over long tables: the two-kernel select gives each
    pair up to 1024 threads, and a table longer than the select's LDS key buffer (6144
    keys) is ranked from the stored keys; an exact tie is planted in the first
    sequence, and K spans one block, a few hundred and more than half the table."""
    monkeypatch.setenv("GPKV_QUEST_SELECT_PATH", "two_kernel")
    w = workloads.random_case(360 + len(ctx), batch=len(ctx), num_q_heads=4 * Hkv,
                              num_kv_heads=Hkv, head_dim=128, block_size=16, context_lens=ctx)
    omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    s = oracle.quest_block_scores(w.query, omin, omax, w.block_tables, w.context_lens, 16, 0, 0)
    a = int(np.argmax(s))
    later = int(s.size - 1 if a != s.size - 1 else s.size - 2)
    kc = w.key_cache.copy()
    kc[int(w.block_tables[0, later])] = kc[int(w.block_tables[0, a])]
    w.key_cache = kc
    nb0 = (ctx[0] + 15) // 16
    for K in (1, 300, nb0 // 2 + 7):
        _, got, exp = _topk_case(w, K)
        assert np.array_equal(got, exp), K


def test_batch_above_balanced_table_uses_split_schedule():
    """4200 sequences (more than the balanced schedule's 4096-sequence prefix): the
    dense, sparse, select and one-call Quest paths fall back to their split or
    two-kernel forms and still match the oracle; multi-token queries refuse the batch
    with UNSUPPORTED."""
    rng = np.random.default_rng(909)
    B = 4200
    ctx = rng.integers(0, 41, size=B).astype(np.int32)
    w = workloads.random_case(909, batch=B, num_q_heads=8, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=ctx)
    d = Dev(w)
    out = _dense(d, w).cpu().numpy()
    seqs = sorted({int(np.argmax(ctx)), int(np.argmin(ctx)), 0, 1, 4096, 4097, B - 1})
    ref = oracle.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                        w.context_lens, w.scale, seqs=seqs)
    assert max_abs(out[seqs], ref[seqs]) <= ATOL
    assert (out[ctx == 0] == 0).all()
    kmin, kmax = _meta(d, w)
    K = 2
    sel = gp.quest_select_topk(d.q, kmin, kmax, d.bt, d.ctx, block_size=16, topk_blocks=K,
                               max_context_len=w.max_context_len)
    omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    osel = oracle.quest_select_topk(w.query[seqs], omin, omax, w.block_tables[seqs],
                                    w.context_lens[seqs], 16, K)
    assert np.array_equal(sel.cpu().numpy()[seqs], osel)
    sp = _sparse(d, w, sel).cpu().numpy()
    oref = oracle.sparse_paged_attention_decode(w.query[seqs], w.key_cache, w.value_cache,
                                                w.block_tables[seqs], w.context_lens[seqs], osel,
                                                w.scale)
    assert max_abs(sp[seqs], oref) <= ATOL
    qd_out, qd_sel = gp.quest_decode(d.q, d.kc, d.vc, kmin, kmax, d.bt, d.ctx, topk_blocks=K,
                                     max_context_len=w.max_context_len, scale=float(w.scale))
    assert torch.equal(qd_sel, sel)
    assert max_abs(qd_out.cpu().numpy()[seqs], oref) <= ATOL
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(gp.GpkvError) as exc:
        gp.paged_attention_varlen(d.q, d.kc, d.vc, d.bt, d.ctx, cu, max_q_len=1,
                                  max_context_len=w.max_context_len, scale=float(w.scale))
    assert exc.value.status == -3
