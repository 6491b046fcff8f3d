"""GPU parity of Quest over E4M3 caches against the CPU oracle.

The metadata holds the codes of each channel's smallest and largest key code value
over a block's valid rows; the block score is the Quest bound on the code values
(the per-KV-head key scale is one positive factor for every block of a head, so it
leaves the selection unchanged). Source: "Ascend Kernel-to-Serving Pipeline",
section "Quest Sparse Attention", over the FP8 cache of the TileLang chapter's KV
quantisation lever.

Bars: metadata equal to the oracle's by value (a zero extreme may be stored as
either zero code), cache codes and Top-K ids bit-exact, attention within max-abs
2e-3 of the float64 oracle evaluated on the oracle's own codes and selection.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import Dev, before_write_lens, max_abs, to_dev, workload
from test_fp8_gpu import Fp8Case, _full_case

pytestmark = pytest.mark.gpu
ATOL = 2e-3
U8 = torch.uint8
CODE_SENTINEL = 0x35   # fills metadata rows no call should touch (E4M3 0.8125)


def code_meta_equal(got, exp) -> bool:
    """Codes equal, except the two zero codes (0x00 and 0x80) count as equal."""
    g = np.array(got, copy=True)
    e = np.array(exp, copy=True)
    g[g == 0x80] = 0
    e[e == 0x80] = 0
    return np.array_equal(g, e)


def _referenced(w):
    bs = w.block_size
    parts = [w.block_tables[b, :-(-int(L) // bs)] for b, L in enumerate(w.context_lens) if L > 0]
    return np.unique(np.concatenate(parts)) if parts else np.zeros(0, np.int64)


def _meta_tensors(w):
    kmin = torch.full((w.num_blocks, w.num_kv_heads, w.head_dim), CODE_SENTINEL, dtype=U8,
                      device="cuda")
    return kmin, torch.full_like(kmin, CODE_SENTINEL)


def _gpu_meta(c, lens=None, last_block_only=False, kmin=None, kmax=None):
    """The GPU's code metadata of the case's GPU-written key codes."""
    w = c.w
    if kmin is None:
        kmin, kmax = _meta_tensors(w)
    ctx = c.d.ctx if lens is None else to_dev(lens, torch.int32)
    gp.quest_block_metadata_fp8(c.kc, c.d.bt, ctx, kmin, kmax, max_context_len=w.max_context_len,
                                last_block_only=last_block_only)
    return kmin, kmax


def _check_meta(w, kmin, kmax, omin, omax):
    ref = _referenced(w)
    gmin, gmax = kmin.cpu().numpy(), kmax.cpu().numpy()
    assert code_meta_equal(gmin[ref], omin[ref]), "key_min codes differ from the oracle"
    assert code_meta_equal(gmax[ref], omax[ref]), "key_max codes differ from the oracle"
    rest = np.setdiff1d(np.arange(w.num_blocks), ref)
    assert (gmin[rest] == CODE_SENTINEL).all() and (gmax[rest] == CODE_SENTINEL).all(), \
        "metadata of unreferenced blocks was written"


@functools.lru_cache(maxsize=None)
def _oracle_meta(config):
    w, c = workload(config), _full_case(config)
    return oracle.quest_block_metadata_fp8(c.okc, w.block_tables, w.context_lens, w.block_size)


@functools.lru_cache(maxsize=None)
def _oracle_sel(config, K):
    w = workload(config)
    omin, omax = _oracle_meta(config)
    return oracle.quest_select_topk_fp8(w.query, omin, omax, w.block_tables, w.context_lens,
                                        w.block_size, K)


# ---------------------------------------------------------------------------
# Metadata
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("config", [1, 3, 4, 5])
def test_fp8_meta_config(config):
    """Whole-pool E4M3 caches written by the GPU; metadata of every referenced block."""
    w, c = workload(config), _full_case(config)
    kmin, kmax = _gpu_meta(c)
    torch.cuda.synchronize()
    _check_meta(w, kmin, kmax, *_oracle_meta(config))


def _all_codes_case(seed, Hq, Hkv, D, bs, ctx):
    """Random finite E4M3 codes over the whole range (both zeros, +-448 included) as
    the key cache, the rows past each context holding +-448; the values cache is
    random codes too (scales 1)."""
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv,
                              head_dim=D, block_size=bs, context_lens=ctx)
    rng = np.random.default_rng(seed)
    finite = np.array([x for x in range(256) if x not in (0x7F, 0xFF)], np.uint8)
    kc = rng.choice(finite, size=w.key_cache.shape).astype(np.uint8)
    zeros = rng.random(kc.shape) < 0.05                     # many exact zeros of both signs
    kc[zeros] = rng.choice(np.array([0x00, 0x80], np.uint8), size=int(zeros.sum()))
    for b, L in enumerate(ctx):
        if L % bs:
            pb = int(w.block_tables[b, L // bs])
            kc[pb, L % bs:, :, ::2] = 0x7E
            kc[pb, L % bs:, :, 1::2] = 0xFE
    vc = rng.choice(finite, size=w.key_cache.shape).astype(np.uint8)
    return w, kc, vc


class CodeCase:
    """A case whose E4M3 caches are given codes (the same on both sides)."""

    def __init__(self, w, kc, vc, ks=None, vs=None):
        self.w, self.seqs = w, list(range(w.batch))
        self.d = Dev(w)
        self.okc, self.ovc = kc, vc
        Hkv = w.num_kv_heads
        self.ks = np.ones(Hkv, np.float32) if ks is None else np.asarray(ks, np.float32)
        self.vs = np.ones(Hkv, np.float32) if vs is None else np.asarray(vs, np.float32)
        self.kc = torch.from_numpy(kc).cuda()
        self.vc = torch.from_numpy(vc).cuda()
        self.d_ks = to_dev(self.ks, torch.float32)
        self.d_vs = to_dev(self.vs, torch.float32)


CODE_CASES = [
    # seed, Hq, Hkv, D, bs, ctx
    (901, 4, 1, 64, 16, [1, 15, 16, 17, 100]),
    (902, 28, 4, 128, 16, [2049, 31, 700]),
    (903, 16, 8, 128, 128, [129, 1, 3000]),
    (904, 14, 2, 64, 32, [33, 64, 65, 1000]),
]


@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx", CODE_CASES)
def test_fp8_meta_all_codes(seed, Hq, Hkv, D, bs, ctx):
    w, kc, vc = _all_codes_case(seed, Hq, Hkv, D, bs, ctx)
    c = CodeCase(w, kc, vc)
    kmin, kmax = _gpu_meta(c)
    torch.cuda.synchronize()
    _check_meta(w, kmin, kmax,
                *oracle.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, bs))


def test_fp8_meta_last_block_only():
    """Step mode writes each sequence's last block only, equal to the full build there."""
    w, kc, vc = _all_codes_case(905, 8, 2, 128, 16, [1, 16, 17, 300, 47])
    c = CodeCase(w, kc, vc)
    kmin, kmax = _gpu_meta(c, last_block_only=True)
    torch.cuda.synchronize()
    base = np.full((w.num_blocks, 2, 128), CODE_SENTINEL, np.uint8)
    omin, omax = oracle.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, 16,
                                                 last_block_only=True, key_min=base, key_max=base)
    assert code_meta_equal(kmin.cpu().numpy(), omin) and code_meta_equal(kmax.cpu().numpy(), omax)


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------

SEL_CONFIGS = [(1, 3), (3, 64), (4, 256), (5, 32)]


@pytest.mark.parametrize("path", ["fused", "two_kernel"])
@pytest.mark.parametrize("config,K", SEL_CONFIGS)
def test_fp8_select_config(config, K, path, monkeypatch):
    monkeypatch.setenv("GPKV_QUEST_SELECT_PATH", path)
    w, c = workload(config), _full_case(config)
    kmin, kmax = _gpu_meta(c)
    sel = gp.quest_select_topk_fp8(c.d.q, kmin, kmax, c.d.bt, c.d.ctx, block_size=w.block_size,
                                   topk_blocks=K, max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), _oracle_sel(config, K)), "selection differs"


@pytest.mark.parametrize("path", ["fused", "two_kernel"])
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx", CODE_CASES)
def test_fp8_select_all_codes(seed, Hq, Hkv, D, bs, ctx, path, monkeypatch):
    """Metadata over every code (negative extremes, zeros of both signs) and K below,
    at and above the block counts."""
    monkeypatch.setenv("GPKV_QUEST_SELECT_PATH", path)
    w, kc, vc = _all_codes_case(seed, Hq, Hkv, D, bs, ctx)
    c = CodeCase(w, kc, vc)
    kmin, kmax = _gpu_meta(c)
    omin, omax = oracle.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, bs)
    for K in (1, 2, 7, 200):
        sel = gp.quest_select_topk_fp8(c.d.q, kmin, kmax, c.d.bt, c.d.ctx, block_size=bs,
                                       topk_blocks=K, max_context_len=w.max_context_len)
        exp = oracle.quest_select_topk_fp8(w.query, omin, omax, w.block_tables, w.context_lens,
                                           bs, K)
        assert np.array_equal(sel.cpu().numpy(), exp), K


@pytest.mark.parametrize("path", ["fused", "two_kernel"])
def test_fp8_select_tie_goes_to_lower_block(path, monkeypatch):
    """Two blocks of one sequence with the same key codes tie; with room for one of them
    the lower logical block is kept."""
    monkeypatch.setenv("GPKV_QUEST_SELECT_PATH", path)
    w, kc, vc = _all_codes_case(906, 4, 1, 128, 16, [64])
    omin, omax = oracle.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, 16)
    s = oracle.quest_block_scores_fp8(w.query, omin, omax, w.block_tables, w.context_lens, 16, 0, 0)
    best = int(np.argmax(s))
    later = max(lb for lb in range(4) if lb != best)
    kc[int(w.block_tables[0, later])] = kc[int(w.block_tables[0, best])]
    c = CodeCase(w, kc, vc)
    kmin, kmax = _gpu_meta(c)
    sel = gp.quest_select_topk_fp8(c.d.q, kmin, kmax, c.d.bt, c.d.ctx, block_size=16,
                                   topk_blocks=1, max_context_len=64)
    torch.cuda.synchronize()
    assert int(sel.cpu()[0, 0, 0]) == min(best, later)


# ---------------------------------------------------------------------------
# The Quest decode step over E4M3 caches
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def _sparse_ref(config, K):
    w, c = workload(config), _full_case(config)
    return oracle.sparse_paged_attention_decode_fp8(w.query, c.okc, c.ovc, c.ks, c.vs,
                                                    w.block_tables, w.context_lens,
                                                    _oracle_sel(config, K), w.scale)


@pytest.mark.parametrize("path", ["auto", "fused", "separate"])
@pytest.mark.parametrize("config,K", SEL_CONFIGS)
def test_fp8_quest_decode_config(config, K, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("GPKV_QUEST_DECODE_PATH", path)
    w, c = workload(config), _full_case(config)
    kmin, kmax = _gpu_meta(c)
    out, sel = gp.quest_decode_fp8(c.d.q, c.kc, c.vc, c.d_ks, c.d_vs, kmin, kmax, c.d.bt, c.d.ctx,
                                   topk_blocks=K, max_context_len=w.max_context_len,
                                   scale=float(w.scale))
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), _oracle_sel(config, K)), "selection differs"
    err = max_abs(out.cpu().numpy(), _sparse_ref(config, K))
    print(f"config {config} K={K} path={path}: FP8 Quest max-abs {err:.3e} over {w.batch} seqs")
    assert err <= ATOL


def _decode_check(c, K):
    w = c.w
    kmin, kmax = _gpu_meta(c)
    out, sel = gp.quest_decode_fp8(c.d.q, c.kc, c.vc, c.d_ks, c.d_vs, kmin, kmax, c.d.bt, c.d.ctx,
                                   topk_blocks=K, max_context_len=w.max_context_len,
                                   scale=float(w.scale))
    torch.cuda.synchronize()
    omin, omax = oracle.quest_block_metadata_fp8(c.okc, w.block_tables, w.context_lens,
                                                 w.block_size)
    osel = oracle.quest_select_topk_fp8(w.query, omin, omax, w.block_tables, w.context_lens,
                                        w.block_size, K)
    assert np.array_equal(sel.cpu().numpy(), osel), "selection differs"
    ref = oracle.sparse_paged_attention_decode_fp8(w.query, c.okc, c.ovc, c.ks, c.vs,
                                                   w.block_tables, w.context_lens, osel, w.scale)
    err = max_abs(out.cpu().numpy(), ref)
    print(f"{w.name} K={K}: FP8 Quest max-abs {err:.3e}")
    assert err <= ATOL
    for b, L in enumerate(w.context_lens):
        if L == 0:
            assert (out.cpu().numpy()[b] == 0).all()


QD_CASES = [
    # seed, Hq, Hkv, D, bs, ctx, K (contexts of 0 and 1, ragged last blocks, K above nb)
    (911, 28, 4, 128, 16, [900, 33, 0, 2500, 1], 12),
    (912, 16, 1, 128, 64, [129, 2048, 4097], 1),
    (913, 14, 2, 64, 128, [257, 1, 700, 3000], 5),
    (914, 8, 1, 64, 16, [40960, 16], 256),
]


@pytest.mark.parametrize("path", ["fused", "separate"])
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx,K", QD_CASES)
def test_fp8_quest_decode_random(seed, Hq, Hkv, D, bs, ctx, K, path, monkeypatch):
    monkeypatch.setenv("GPKV_QUEST_DECODE_PATH", path)
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=ctx)
    _decode_check(Fp8Case(w, list(range(w.batch))), K)


@pytest.mark.parametrize("path", ["fused", "separate"])
def test_fp8_quest_decode_all_codes_scaled(path, monkeypatch):
    """Codes over the whole range with per-head K and V scales that differ."""
    monkeypatch.setenv("GPKV_QUEST_DECODE_PATH", path)
    w, kc, vc = _all_codes_case(915, 28, 4, 128, 16, [2049, 31, 700])
    c = CodeCase(w, kc, vc, ks=[0.002, 0.01, 0.0005, 0.004], vs=[0.01, 0.002, 0.02, 0.001])
    _decode_check(c, 9)


# ---------------------------------------------------------------------------
# The write path with the code metadata fold, and the step in one call
# ---------------------------------------------------------------------------

def _pre_write_meta(c):
    """GPU metadata over the contexts before this step's write (the fold's starting
    point) and the oracle's counterpart."""
    w = c.w
    lens = before_write_lens(w)
    kmin, kmax = _gpu_meta(c, lens=lens)
    base = np.full((w.num_blocks, w.num_kv_heads, w.head_dim), CODE_SENTINEL, np.uint8)
    pmin, pmax = oracle.quest_block_metadata_fp8(c.okc, w.block_tables, lens, w.block_size,
                                                 key_min=base, key_max=base)
    return kmin, kmax, pmin, pmax


def _oracle_write(c):
    w = c.w
    return oracle.reshape_and_cache_fp8(c.okc, c.ovc, w.new_key, w.new_value, w.slot_mapping,
                                        w.block_size, c.ks, c.vs)


def _check_codes(c, kc, vc, ek, ev):
    ref = _referenced(c.w)
    assert np.array_equal(kc.cpu().numpy()[ref], ek[ref]), "key codes differ from the oracle"
    assert np.array_equal(vc.cpu().numpy()[ref], ev[ref]), "value codes differ from the oracle"


def test_fp8_write_with_meta_fold():
    """reshape_and_cache_fp8_quest of each sequence's newest token: codes as the FP8
    write, metadata as the oracle's rebuild of each written block (new tokens at row 0
    of a block, at its last row and in between; one slot negative)."""
    w = workloads.random_case(921, batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128,
                              block_size=16, context_lens=[1, 16, 17, 33, 100, 64],
                              num_tokens=6, neg_slots=1)
    c = Fp8Case(w, list(range(w.batch)))
    kmin, kmax, pmin, pmax = _pre_write_meta(c)
    kc, vc = c.kc.clone(), c.vc.clone()
    gp.reshape_and_cache_fp8_quest(c.d.nk, c.d.nv, kc, vc, c.d_ks, c.d_vs, kmin, kmax, c.d.slots)
    torch.cuda.synchronize()
    ek, ev = _oracle_write(c)
    _check_codes(c, kc, vc, ek, ev)
    emin, emax = oracle.quest_block_metadata_fp8(ek, w.block_tables, w.context_lens, 16,
                                                 key_min=pmin, key_max=pmax)
    assert code_meta_equal(kmin.cpu().numpy(), emin), "key_min differs from the oracle chain"
    assert code_meta_equal(kmax.cpu().numpy(), emax), "key_max differs from the oracle chain"


def _append_check(c, K, path, monkeypatch):
    """quest_decode_fp8_append against the oracle chain: FP8 write, code metadata of the
    written caches, Top-K, FP8 sparse attention."""
    if path != "auto":
        monkeypatch.setenv("GPKV_QUEST_DECODE_PATH", path)
    w = c.w
    assert w.num_tokens == w.batch, "decode append writes token b for sequence b"
    kmin, kmax, _, _ = _pre_write_meta(c)
    kc, vc = c.kc.clone(), c.vc.clone()
    out, sel = gp.quest_decode_fp8_append(c.d.q, c.d.nk, c.d.nv, kc, vc, c.d_ks, c.d_vs, kmin,
                                          kmax, c.d.slots, c.d.bt, c.d.ctx, topk_blocks=K,
                                          max_context_len=w.max_context_len, scale=float(w.scale))
    torch.cuda.synchronize()
    ek, ev = _oracle_write(c)
    _check_codes(c, kc, vc, ek, ev)
    omin, omax = oracle.quest_block_metadata_fp8(ek, w.block_tables, w.context_lens, w.block_size)
    ref = _referenced(w)
    assert code_meta_equal(kmin.cpu().numpy()[ref], omin[ref]), "key_min differs"
    assert code_meta_equal(kmax.cpu().numpy()[ref], omax[ref]), "key_max differs"
    osel = oracle.quest_select_topk_fp8(w.query, omin, omax, w.block_tables, w.context_lens,
                                        w.block_size, K)
    assert np.array_equal(sel.cpu().numpy(), osel), "selection differs from the oracle"
    exp = oracle.sparse_paged_attention_decode_fp8(w.query, ek, ev, c.ks, c.vs, w.block_tables,
                                                   w.context_lens, osel, w.scale)
    err = max_abs(out.cpu().numpy(), exp)
    print(f"{w.name} K={K} path={path}: FP8 Quest append max-abs {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("config,K,path", [(1, 3, "auto"), (1, 5, "separate"), (3, 64, "auto"),
                                           (3, 64, "separate"), (5, 32, "auto")])
def test_fp8_quest_append_config(config, K, path, monkeypatch):
    _append_check(_full_case(config), K, path, monkeypatch)


APPEND_CASES = [
    (931, 28, 4, 128, 16, [900, 33, 2500, 17, 1, 700], 12, 1),
    (932, 16, 1, 128, 64, [129, 2048, 4097], 1, 0),
    (933, 14, 2, 64, 128, [257, 1, 700, 3000], 5, 1),
]


@pytest.mark.parametrize("path", ["fused", "separate"])
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx,K,neg", APPEND_CASES)
def test_fp8_quest_append_random(seed, Hq, Hkv, D, bs, ctx, K, neg, path, monkeypatch):
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=ctx, num_tokens=len(ctx), neg_slots=neg)
    _append_check(Fp8Case(w, list(range(w.batch))), K, path, monkeypatch)


@pytest.mark.parametrize("path", ["fused", "separate"])
def test_fp8_quest_append_spiked_new_token(path, monkeypatch):
    """New keys three times each head's query (one query head per KV head): the fold moves
    the selection (checked on the oracle against stale metadata) and the new token
    carries much of its sequence's softmax."""
    w = workloads.random_case(941, batch=3, num_q_heads=4, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=[3000, 700, 40], num_tokens=3)
    q = oracle.bf16_to_f64(w.query)
    w.new_key[...] = workloads.bf16_bits((3.0 * q).astype(np.float32))
    c = Fp8Case(w, list(range(w.batch)))
    ek, _ = _oracle_write(c)
    lens = before_write_lens(w)
    smin, smax = oracle.quest_block_metadata_fp8(c.okc, w.block_tables, lens, 16)
    gmin, gmax = oracle.quest_block_metadata_fp8(ek, w.block_tables, w.context_lens, 16)
    stale = oracle.quest_select_topk_fp8(w.query, smin, smax, w.block_tables, w.context_lens, 16, 4)
    good = oracle.quest_select_topk_fp8(w.query, gmin, gmax, w.block_tables, w.context_lens, 16, 4)
    assert not np.array_equal(stale, good), "the case does not depend on the fold"
    _append_check(c, 4, path, monkeypatch)


def test_fp8_quest_batch_above_balanced_table():
    """4200 sequences (past the balanced schedule's 4096-sequence prefix): the FP8
    selection and the one-call FP8 Quest step take their two-kernel and split forms and
    match the oracle on sampled sequences (the oracle's codes cover those sequences'
    blocks)."""
    rng = np.random.default_rng(951)
    B = 4200
    ctx = rng.integers(0, 41, size=B).astype(np.int32)
    w = workloads.random_case(951, batch=B, num_q_heads=8, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=ctx)
    seqs = sorted({int(np.argmax(ctx)), int(np.argmin(ctx)), 0, 1, 4096, 4097, B - 1})
    c = Fp8Case(w, seqs)
    kmin, kmax = _gpu_meta(c)
    K = 2
    sel = gp.quest_select_topk_fp8(c.d.q, kmin, kmax, c.d.bt, c.d.ctx, block_size=16,
                                   topk_blocks=K, max_context_len=w.max_context_len)
    out, qsel = gp.quest_decode_fp8(c.d.q, c.kc, c.vc, c.d_ks, c.d_vs, kmin, kmax, c.d.bt,
                                    c.d.ctx, topk_blocks=K, max_context_len=w.max_context_len,
                                    scale=float(w.scale))
    torch.cuda.synchronize()
    bt, cl = w.block_tables[seqs], w.context_lens[seqs]
    omin, omax = oracle.quest_block_metadata_fp8(c.okc, bt, cl, 16)
    osel = oracle.quest_select_topk_fp8(w.query[seqs], omin, omax, bt, cl, 16, K)
    assert np.array_equal(sel.cpu().numpy()[seqs], osel), "selection differs"
    assert torch.equal(qsel, sel), "the one-call step selected differently"
    ref = oracle.sparse_paged_attention_decode_fp8(w.query[seqs], c.okc, c.ovc, c.ks, c.vs, bt,
                                                   cl, osel, w.scale)
    o = out.cpu().numpy()
    assert max_abs(o[seqs], ref) <= ATOL
    assert (o[ctx == 0] == 0).all()
