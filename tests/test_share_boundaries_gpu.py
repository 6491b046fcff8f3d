"""Parity at the schedules' seams: spike tokens where work is cut between workgroups
and waves, on the full-size workloads, in the schedule each call takes by default.

At full size the 2e-3 bar alone cannot see a lost or doubled token: one token among
thousands carries a weight of about 1e-4. So tokens whose keys point along their
group's summed query are planted exactly where the schedule cuts the work:

  - dense (balanced schedule, one workgroup per CU): the flattened space of
    (sequence, 16-token sub-tile), where every non-empty sequence opens with
    SEG_COST sub-tiles of no work, is shared out as [wg*S/N, (wg+1)*S/N); a spike
    sits on the first token of every share and on the last token of the share
    before it;
  - sparse, balanced schedule (the 8-KV-head ragged batch): the same rule over the
    sub-tiles of each sequence's selected blocks, in list order;
  - sparse, one workgroup per (sequence, KV head) (the 8K-average batch): its four
    waves take [w*T/4, (w+1)*T/4) of the pair's 32-token tiles;
  - the one-launch Quest decode (the 8K-average batch): its workgroup of eight waves
    selects the pair's blocks, then wave w takes [w*T/8, (w+1)*T/8) of the selected
    32-token tiles;

plus the first and last token of every sequence. Each spike outweighs the rest of
its sequence many times over, so the spikes share the softmax weight among
themselves: dropping or doubling one moves the output by O(0.1) or more, which the
tests check on the oracle before comparing. The work split used to place the spikes
restates the library's host-side rule (one workgroup per compute unit unless a
share would exceed the per-workgroup table).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import BF, Dev, fp8_codes, max_abs, oracle_selection, to_dev, workload

pytestmark = pytest.mark.gpu
ATOL = 2e-3
SPIKE_SCORE = 20.0      # scale * q.k of a spike for the median head of its group
MAX_SUB_PER_WG = 2048   # dense balanced schedule: most sub-tiles per workgroup
BAL_TAB = 4096          # sparse balanced schedule: table entries per workgroup
SEG_COST = 2            # balanced schedules: cost of starting a sequence, in sub-tiles
DIRECT_WAVES = 4        # waves of the one-workgroup-per-(sequence, KV head) sparse path
QUEST_WAVES = 8         # waves of the one-launch Quest decode's workgroup


def _cus() -> int:
    return int(torch.cuda.get_device_properties(0).multi_processor_count)


def _balanced_workgroups(max_sub: int, share_max: int, batch: int) -> int:
    n = max(_cus(), -(-(max_sub + batch * SEG_COST) // share_max))
    return max(1, min(n, max_sub))


def _cuts(work: np.ndarray, nwg: int):
    """(item, first sub-tile of a share inside it) for every share boundary of the
    flattened work (sub-tiles per item, each non-empty item opening with SEG_COST
    sub-tiles of no work), as the balanced schedule draws them."""
    work = work.astype(np.int64)
    cost = work + np.where(work > 0, SEG_COST, 0)
    pre = np.concatenate([[0], np.cumsum(cost)])
    S = int(pre[-1])
    out = []
    for wg in range(1, nwg):
        s0 = wg * S // nwg
        if s0 >= S or s0 == (wg - 1) * S // nwg:
            continue
        b = int(np.searchsorted(pre, s0, side="right") - 1)
        out.append((b, max(0, s0 - int(pre[b]) - SEG_COST)))
    return out


def _spike_keys(w) -> np.ndarray:
    """Per (sequence, KV head): gamma times the sum of the group's queries, with gamma
    putting the median head's scaled score at SPIKE_SCORE (bf16 bits)."""
    q = oracle.bf16_to_f64(w.query)
    G = w.num_q_heads // w.num_kv_heads
    sc = float(np.float32(w.scale))
    keys = np.zeros((w.batch, w.num_kv_heads, w.head_dim), np.uint16)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            qg = q[b, g * G:(g + 1) * G]
            a = qg.sum(axis=0)
            med = float(np.median(sc * (qg @ a)))
            assert med > 0
            keys[b, g] = workloads.bf16_bits((SPIKE_SCORE / med * a).astype(np.float32))
    return keys


def _plant(w, spikes):
    """A copy of the workload with the spikes (b, g, t) written into its pool: the
    spike key of (b, g), and a value row of its own (4 x N(0, 1))."""
    keys = _spike_keys(w)
    kc, vc = w.key_cache.copy(), w.value_cache.copy()
    rng = np.random.default_rng(4242)
    bs = w.block_size
    for b, g, t in sorted(spikes):
        pb, row = int(w.block_tables[b, t // bs]), t % bs
        kc[pb, row, g] = keys[b, g]
        vc[pb, row, g] = workloads.bf16_bits(4.0 * rng.standard_normal(w.head_dim).astype(np.float32))
    return dataclasses.replace(w, key_cache=kc, value_cache=vc)


def _dense_spikes(w):
    ctx = w.context_lens.astype(np.int64)
    work = (ctx + 15) // 16
    nwg = _balanced_workgroups(int(w.batch * ((w.max_context_len + 15) // 16)), MAX_SUB_PER_WG,
                               w.batch)
    pos = set()
    for b, u in _cuts(work, nwg):
        pos.add((b, 16 * u))
        pos.add((b, 16 * u - 1) if u > 0 else (b - 1, int(ctx[b - 1]) - 1))
    for b in range(w.batch):
        if ctx[b] > 0:
            pos.update({(b, 0), (b, int(ctx[b]) - 1)})
    pos = {(b, t) for b, t in pos if b >= 0 and 0 <= t < ctx[b]}
    return nwg, {(b, g, t) for b, t in pos for g in range(w.num_kv_heads)}


def _selected_token(sel_row, e, row, ctx, bs):
    """Token at row `row` of the e-th selected block, or None past the context."""
    t = int(sel_row[e]) * bs + row
    return t if t < ctx else None


def _sparse_balanced_spikes(w, sel, K):
    bs, spb = w.block_size, w.block_size // 16
    ctx = w.context_lens.astype(np.int64)
    nsel = np.minimum(K, -(-ctx // bs))
    nwg = _balanced_workgroups(int(w.batch * K * spb), (BAL_TAB // w.num_kv_heads - 2) * spb,
                               w.batch)
    spikes = set()
    for b, u in _cuts(nsel * spb, nwg):
        for g in range(w.num_kv_heads):
            for uu, row_in in ((u, 0), (u - 1, 15)):
                if uu < 0:
                    continue
                t = _selected_token(sel[b, g], uu // spb, (uu % spb) * 16 + row_in, ctx[b], bs)
                if t is None:   # a sub-tile past the context: its last valid token instead
                    t = int(ctx[b]) - 1 if int(sel[b, g, uu // spb]) * bs <= ctx[b] - 1 else None
                if t is not None:
                    spikes.add((b, g, t))
    return nwg, spikes


def _direct_spikes(w, sel, K, waves=DIRECT_WAVES):
    bs, spb = w.block_size, w.block_size // 16
    ctx = w.context_lens.astype(np.int64)
    spikes = set()
    for b in range(w.batch):
        n = int(min(K, -(-ctx[b] // bs)))
        if n == 0:
            continue
        n_tiles = (n * spb + 1) // 2
        for g in range(w.num_kv_heads):
            for wave in range(1, waves):
                u = 2 * (wave * n_tiles // waves)
                for uu, row_in in ((u, 0), (u - 1, 15)):
                    if 0 <= uu < n * spb:
                        t = _selected_token(sel[b, g], uu // spb, (uu % spb) * 16 + row_in,
                                            ctx[b], bs)
                        if t is not None:
                            spikes.add((b, g, t))
            first = int(sel[b, g, 0]) * bs
            last = min(int(sel[b, g, n - 1]) * bs + bs, int(ctx[b])) - 1
            spikes.update({(b, g, first), (b, g, last)})
    return spikes


def _assert_drop_is_visible(w, spikes, attend):
    """Removing one spike of a sequence (its bits restored) moves that sequence's
    oracle output by far more than the bar: the planted tokens are discriminating."""
    base = workload(w.config)
    b, g, t = sorted(spikes)[len(spikes) // 2]
    w2 = dataclasses.replace(w, key_cache=w.key_cache.copy(), value_cache=w.value_cache.copy())
    pb, row = int(w.block_tables[b, t // w.block_size]), t % w.block_size
    w2.key_cache[pb, row, g] = base.key_cache[pb, row, g]
    w2.value_cache[pb, row, g] = base.value_cache[pb, row, g]
    moved = max_abs(attend(w, [b])[b], attend(w2, [b])[b])
    assert moved > 50 * ATOL, f"dropping spike {(b, g, t)} moves the output by only {moved:.2e}"


def _dense_oracle(w, seqs=None):
    return oracle.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                         w.context_lens, w.scale, seqs=seqs)


@pytest.mark.parametrize("config", [3, 5])
def test_dense_spikes_at_balanced_share_boundaries(config):
    w0 = workload(config)
    nwg, spikes = _dense_spikes(w0)
    w = _plant(w0, spikes)
    _assert_drop_is_visible(w, spikes, _dense_oracle)
    d = Dev(w)
    out = gp.paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx, max_context_len=w.max_context_len,
                                    scale=float(w.scale)).cpu().numpy()
    err = max_abs(out, _dense_oracle(w))
    print(f"config {config}: {len(spikes)} spikes over {nwg} shares; dense max-abs {err:.3e}")
    assert err <= ATOL


def test_fp8_dense_spikes_at_balanced_share_boundaries():
    """The E4M3 instance of the dense kernel at the same seams (8K-average batch)."""
    w0 = workload(3)
    nwg, spikes = _dense_spikes(w0)
    w = _plant(w0, spikes)

    def scales(bits):
        x = oracle.bf16_to_f64(bits)
        return (np.abs(x).max(axis=(0, 1, 3)) / 256.0).clip(min=1e-3).astype(np.float32)
    ks, vs = scales(w.key_cache), scales(w.value_cache)
    okc, ovc = fp8_codes(w.key_cache, ks), fp8_codes(w.value_cache, vs)
    d = Dev(w)
    NB, bs, Hkv, D = w.key_cache.shape
    kc8 = torch.empty((NB, bs, Hkv, D), dtype=torch.uint8, device="cuda")
    vc8 = torch.empty_like(kc8)
    d_ks, d_vs = to_dev(ks, torch.float32), to_dev(vs, torch.float32)
    gp.reshape_and_cache_fp8(d.kc.view(NB * bs, Hkv, D), d.vc.view(NB * bs, Hkv, D), kc8, vc8,
                             d_ks, d_vs, torch.arange(NB * bs, dtype=torch.int64, device="cuda"))
    assert np.array_equal(kc8.cpu().numpy(), okc) and np.array_equal(vc8.cpu().numpy(), ovc)

    def attend(wx, seqs=None):
        kq = okc if wx is w else fp8_codes(wx.key_cache, ks)
        vq = ovc if wx is w else fp8_codes(wx.value_cache, vs)
        return oracle.paged_attention_decode_fp8(wx.query, kq, vq, ks, vs, wx.block_tables,
                                                 wx.context_lens, wx.scale, seqs=seqs)
    _assert_drop_is_visible(w, spikes, attend)
    out = gp.paged_attention_decode_fp8(d.q, kc8, vc8, d_ks, d_vs, d.bt, d.ctx,
                                        max_context_len=w.max_context_len,
                                        scale=float(w.scale)).cpu().numpy()
    err = max_abs(out, attend(w))
    print(f"FP8: {len(spikes)} spikes over {nwg} shares; dense max-abs {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("config,K", [(5, 32), (3, 64)])
def test_sparse_spikes_at_schedule_seams(config, K):
    """The ragged 8-KV-head batch takes the balanced sparse schedule, the 8K-average
    batch one workgroup per (sequence, KV head): spikes at the seams of each, the
    selection fixed to the oracle's Top-K of the unspiked pool."""
    w0 = workload(config)
    sel = oracle_selection(config, K)
    if config == 5:
        nwg, spikes = _sparse_balanced_spikes(w0, sel, K)
        where = f"{nwg} shares"
    else:
        spikes = _direct_spikes(w0, sel, K)
        where = "wave quarters"
    w = _plant(w0, spikes)

    def attend(wx, seqs=None):
        return oracle.sparse_paged_attention_decode(wx.query, wx.key_cache, wx.value_cache,
                                                    wx.block_tables, wx.context_lens, sel,
                                                    wx.scale, seqs=seqs)
    _assert_drop_is_visible(w, spikes, attend)
    d = Dev(w)
    out = gp.sparse_paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx, to_dev(sel, torch.int32),
                                           max_context_len=w.max_context_len,
                                           scale=float(w.scale)).cpu().numpy()
    err = max_abs(out, attend(w))
    print(f"config {config}: {len(spikes)} spikes at {where}; sparse max-abs {err:.3e}")
    assert err <= ATOL


def test_quest_decode_spikes_at_wave_seams(monkeypatch):
    """The one-launch Quest decode on the 8K-average batch: one 512-thread workgroup per
    (sequence, KV head) selects its blocks and its eight waves take [w*T/8, (w+1)*T/8) of
    the pair's selected 32-token tiles. Spikes sit at those seams of the oracle's
    selection and at each pair's first and last selected token; they only raise the
    scores of selected blocks, so the selection stays the same (checked), and the
    kernel selects and attends by itself."""
    monkeypatch.setenv("GPKV_QUEST_DECODE_PATH", "fused")
    config, K = 3, 64
    w0 = workload(config)
    sel = oracle_selection(config, K)
    spikes = _direct_spikes(w0, sel, K, waves=QUEST_WAVES)
    w = _plant(w0, spikes)
    bs = w.block_size
    omin, omax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, bs)
    assert np.array_equal(
        oracle.quest_select_topk(w.query, omin, omax, w.block_tables, w.context_lens, bs, K), sel)

    def attend(wx, seqs=None):
        return oracle.sparse_paged_attention_decode(wx.query, wx.key_cache, wx.value_cache,
                                                    wx.block_tables, wx.context_lens, sel,
                                                    wx.scale, seqs=seqs)
    _assert_drop_is_visible(w, spikes, attend)
    d = Dev(w)
    kmin = torch.zeros((w.num_blocks, w.num_kv_heads, w.head_dim), dtype=BF, device="cuda")
    kmax = torch.zeros_like(kmin)
    gp.quest_block_metadata(d.kc, d.bt, d.ctx, kmin, kmax, max_context_len=w.max_context_len)
    out, gsel = gp.quest_decode(d.q, d.kc, d.vc, kmin, kmax, d.bt, d.ctx, topk_blocks=K,
                                max_context_len=w.max_context_len, scale=float(w.scale))
    torch.cuda.synchronize()
    assert np.array_equal(gsel.cpu().numpy(), sel), "selection differs from the oracle"
    err = max_abs(out.cpu().numpy(), attend(w))
    print(f"config {config}: {len(spikes)} spikes at the eight wave seams; one-launch Quest "
          f"max-abs {err:.3e}")
    assert err <= ATOL
