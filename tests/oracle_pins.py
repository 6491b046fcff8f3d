"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes an oracle module and raises AssertionError when the oracle
disagrees with a fact that the pages or plain mathematics fix: a pure-Python
brute force written from the definition, torch's CPU scaled-dot-product attention
(a library routine that computes the same textbook operation), closed forms,
invariants, exact rational arithmetic, and hand-worked examples.

The same pins run against mutated copies of the oracle in test_oracle_mutants.py
to show that a plausible slip (a dropped scale, a wrong group index, a flipped
tie rule...) fails at least one of them.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import workloads

TOL = 1e-12


def _dec(bits):
    """bf16 bits -> Python floats, via struct-free integer arithmetic."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _tiny_cases():
    cases = [workloads.make(1)]
    cases.append(workloads.random_case(11, batch=3, num_q_heads=6, num_kv_heads=2, head_dim=64,
                                       block_size=16, context_lens=[1, 17, 50]))
    cases.append(workloads.random_case(12, batch=2, num_q_heads=8, num_kv_heads=4, head_dim=64,
                                       block_size=32, context_lens=[33, 64]))
    return cases


# ---------------------------------------------------------------------------
# ReshapeAndCache
# ---------------------------------------------------------------------------

def pin_write_hand_worked(orc):
    """Slots worked out by hand with block_size 4: 5 -> (1,1), 0 -> (0,0), 15 -> (3,3)."""
    NB, bs, H, D = 4, 4, 1, 2
    kc = np.zeros((NB, bs, H, D), np.uint16)
    vc = np.zeros((NB, bs, H, D), np.uint16)
    key = np.array([[[1, 2]], [[3, 4]], [[5, 6]], [[7, 8]]], np.uint16)
    val = key + 100
    slots = np.array([5, -1, 0, 15], np.int64)
    k2, v2 = orc.reshape_and_cache(kc, vc, key, val, slots, bs)
    ek = np.zeros_like(kc)
    ek[1, 1, 0] = [1, 2]
    ek[0, 0, 0] = [5, 6]
    ek[3, 3, 0] = [7, 8]
    ev = np.zeros_like(vc)
    ev[1, 1, 0] = [101, 102]
    ev[0, 0, 0] = [105, 106]
    ev[3, 3, 0] = [107, 108]
    assert np.array_equal(k2, ek), "key cache after hand-worked write"
    assert np.array_equal(v2, ev), "value cache after hand-worked write"
    assert not kc.any() and not vc.any(), "inputs must not be modified"


def pin_write_config1(orc):
    """The tiny workload (contexts 37 and 80, block size 16): token 0 goes to
    (seq 0, position 36) -> logical block 2, row 4;
    token 1 has slot -1 and changes nothing. Every other byte is untouched."""
    w = workloads.make(1)
    k2, v2 = orc.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                   w.slot_mapping, w.block_size)
    pb = int(w.block_tables[0, 36 // 16])
    assert int(w.slot_mapping[0]) == pb * 16 + 4
    ek = w.key_cache.copy()
    ek[pb, 4] = w.new_key[0]
    ev = w.value_cache.copy()
    ev[pb, 4] = w.new_value[0]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)


def pin_write_negative_skips(orc):
    w = workloads.make(1)
    slots = np.array([-1, -7], np.int64)
    k2, v2 = orc.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value, slots, 16)
    assert np.array_equal(k2, w.key_cache) and np.array_equal(v2, w.value_cache)


# ---------------------------------------------------------------------------
# Dense attention
# ---------------------------------------------------------------------------

def _brute_dense_row(w, b, h):
    """Pure-Python definition: walk the block table token by token."""
    G = w.num_q_heads // w.num_kv_heads
    g = h // G
    bs = w.block_size
    scale = float(w.scale)
    q = _dec(w.query[b, h]).tolist()
    L = int(w.context_lens[b])
    if L == 0:
        return [0.0] * w.head_dim
    scores, vals = [], []
    for t in range(L):
        pb = int(w.block_tables[b][t // bs])
        k = _dec(w.key_cache[pb, t % bs, g]).tolist()
        vals.append(_dec(w.value_cache[pb, t % bs, g]).tolist())
        scores.append(scale * math.fsum(qi * ki for qi, ki in zip(q, k)))
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    z = math.fsum(e)
    return [math.fsum(e[t] * vals[t][c] for t in range(L)) / z for c in range(w.head_dim)]


def pin_dense_brute_force(orc):
    for w in _tiny_cases():
        out = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                         w.context_lens, w.scale)
        for b in range(w.batch):
            for h in range(w.num_q_heads):
                ref = np.array(_brute_dense_row(w, b, h))
                err = np.abs(out[b, h] - ref).max()
                assert err <= TOL, f"{w.name} b={b} h={h} err={err}"


def pin_dense_torch_sdpa(orc):
    """torch CPU scaled_dot_product_attention in float64 with enable_gqa (head h
    reads KV head h // G) on the K/V gathered into contiguous order."""
    import torch
    import torch.nn.functional as F
    for w in _tiny_cases():
        out = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                         w.context_lens, w.scale)
        for b in range(w.batch):
            L = int(w.context_lens[b])
            if L == 0:
                continue
            k = np.stack([_dec(w.key_cache[int(w.block_tables[b][t // w.block_size]), t % w.block_size])
                          for t in range(L)])                  # [L, Hkv, D]
            v = np.stack([_dec(w.value_cache[int(w.block_tables[b][t // w.block_size]), t % w.block_size])
                          for t in range(L)])
            qt = torch.from_numpy(_dec(w.query[b]))[None, :, None, :]       # [1,Hq,1,D]
            kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()    # [1,Hkv,L,D]
            vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
            ref = F.scaled_dot_product_attention(qt, kt, vt, scale=float(w.scale), enable_gqa=True)
            err = np.abs(out[b] - ref[0, :, 0].numpy()).max()
            assert err <= TOL, f"{w.name} b={b} sdpa err={err}"


def pin_dense_closed_forms(orc):
    w = workloads.random_case(21, batch=3, num_q_heads=4, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[1, 40, 23])
    # ctx = 1: the output is the single value row, exactly.
    out = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                     w.context_lens, w.scale)
    pb = int(w.block_tables[0, 0])
    for h in range(4):
        assert np.array_equal(out[0, h], _dec(w.value_cache[pb, 0, h // 2])), "ctx=1 -> v_0"
    # all keys of a sequence equal -> uniform weights -> mean of V.
    kc = w.key_cache.copy()
    for t in range(40):
        kc[int(w.block_tables[1, t // 16]), t % 16] = w.key_cache[int(w.block_tables[1, 0]), 0]
    out = orc.paged_attention_decode(w.query, kc, w.value_cache, w.block_tables, w.context_lens, w.scale)
    for h in range(4):
        vs = [_dec(w.value_cache[int(w.block_tables[1, t // 16]), t % 16, h // 2]) for t in range(40)]
        ref = np.array([math.fsum(v[c] for v in vs) / 40 for c in range(64)])
        assert np.abs(out[1, h] - ref).max() <= TOL, "equal keys -> mean(v)"
    # constant V -> output equals that constant.
    vc = np.full_like(w.value_cache, 0x3FC0)        # bf16 1.5
    out = orc.paged_attention_decode(w.query, w.key_cache, vc, w.block_tables, w.context_lens, w.scale)
    assert np.abs(out - 1.5).max() <= TOL, "constant V"


def pin_dense_scale_and_group(orc):
    """Doubling the query equals doubling the scale (scores are linear in scale*q),
    and moving KV head 1's data onto head 0 only changes the second group's heads."""
    w = workloads.random_case(22, batch=2, num_q_heads=6, num_kv_heads=3, head_dim=64,
                              block_size=16, context_lens=[29, 45])
    out1 = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                      w.context_lens, w.scale)
    ref = np.zeros_like(out1)
    for b in range(2):
        for h in range(6):
            ref[b, h] = _brute_dense_row(w, b, h)
    assert np.abs(out1 - ref).max() <= TOL
    kc = w.key_cache.copy()
    kc[:, :, 1] = kc[:, :, 0]
    vc = w.value_cache.copy()
    vc[:, :, 1] = vc[:, :, 0]
    out2 = orc.paged_attention_decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
    assert np.array_equal(out2[:, [0, 1, 4, 5]], out1[:, [0, 1, 4, 5]]), "heads of groups 0, 2 unchanged"
    assert not np.allclose(out2[:, [2, 3]], out1[:, [2, 3]]), "heads of group 1 read KV head 1"


def _permuted_pool(w, seed):
    """Move every physical block to a new id (data copied along)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_blocks)            # new id of old block i
    kc = np.empty_like(w.key_cache)
    vc = np.empty_like(w.value_cache)
    kc[perm] = w.key_cache
    vc[perm] = w.value_cache
    bt = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    return kc, vc, bt


def pin_dense_permuted_table(orc):
    for w in _tiny_cases():
        out = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                         w.context_lens, w.scale)
        kc, vc, bt = _permuted_pool(w, 5)
        out2 = orc.paged_attention_decode(w.query, kc, vc, bt, w.context_lens, w.scale)
        assert np.array_equal(out, out2), "permuted block table"


def _poison(w, value=0x7FC0):
    """Fill every slot outside some sequence's context with ``value`` bits (NaN)."""
    kc = w.key_cache.copy()
    vc = w.value_cache.copy()
    live = np.zeros(w.key_cache.shape[:2], dtype=bool)
    for b in range(w.batch):
        for t in range(int(w.context_lens[b])):
            live[int(w.block_tables[b, t // w.block_size]), t % w.block_size] = True
    kc[~live] = value
    vc[~live] = value
    return kc, vc


def pin_dense_nan_poison(orc):
    for w in _tiny_cases():
        out = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                         w.context_lens, w.scale)
        kc, vc = _poison(w)
        out2 = orc.paged_attention_decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
        assert np.array_equal(out, out2), "NaN outside the context changed the output"


def pin_dense_empty_context(orc):
    w = workloads.random_case(23, batch=2, num_q_heads=2, num_kv_heads=1, head_dim=64,
                              block_size=16, context_lens=[0, 5])
    out = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                     w.context_lens, w.scale)
    assert np.array_equal(out[0], np.zeros((2, 64))), "ctx = 0 -> zeros"


# ---------------------------------------------------------------------------
# Split-KV combine
# ---------------------------------------------------------------------------

def pin_split_combine_equals_dense(orc):
    w = workloads.random_case(31, batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                              block_size=16, context_lens=[200])
    dense = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                       w.context_lens, w.scale)[0]
    pos = np.arange(200)
    k = orc.bf16_to_f64(orc.gather_sequence(w.key_cache, w.block_tables, 0, pos, 16))[:, 0]
    v = orc.bf16_to_f64(orc.gather_sequence(w.value_cache, w.block_tables, 0, pos, 16))[:, 0]
    q = orc.bf16_to_f64(w.query[0])
    sc = float(w.scale) * 8.0      # sharpen the softmax so the splits' maxima differ a lot
    dense_sharp = orc.split_kv_combine(*orc.split_kv_partials(q, k, v, sc, [(0, 200)]))
    ref = np.array([[_ref_row(q[h], k, v, sc)] for h in range(4)])[:, 0]
    assert np.abs(dense_sharp - ref).max() <= TOL
    for S in (1, 2, 3, 7, 64):
        prop = [(200 * s // S, 200 * (s + 1) // S) for s in range(S)]
        fixed = [(min(200, 32 * s), min(200, 32 * (s + 1))) for s in range(S)] + [(32 * S, 200)]
        for bounds in (prop, fixed):
            got = orc.split_kv_combine(*orc.split_kv_partials(q, k, v, sc, bounds))
            assert np.abs(got - ref).max() <= TOL, f"S={S} split combine"
    got = orc.split_kv_combine(*orc.split_kv_partials(q, k, v, float(w.scale), [(0, 0), (0, 77), (77, 77), (77, 200)]))
    assert np.abs(got - dense).max() <= TOL, "empty splits carry weight 0"


def _ref_row(qh, k, v, sc):
    s = [sc * math.fsum(a * b for a, b in zip(qh, kt)) for kt in k]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = math.fsum(e)
    return [math.fsum(e[t] * v[t][c] for t in range(len(e))) / z for c in range(v.shape[1])]


# ---------------------------------------------------------------------------
# Quest metadata
# ---------------------------------------------------------------------------

def _brute_meta(w):
    NB, bs, H, D = w.key_cache.shape
    kmin = {}
    kmax = {}
    for b in range(w.batch):
        L = int(w.context_lens[b])
        for lb in range(-(-L // bs)):
            pb = int(w.block_tables[b, lb])
            n = min(bs, L - lb * bs)
            for g in range(H):
                for c in range(D):
                    vals = [float(_dec(w.key_cache[pb, t, g, c])) for t in range(n)]
                    kmin[(pb, g, c)] = min(vals)
                    kmax[(pb, g, c)] = max(vals)
    return kmin, kmax


def pin_meta_brute_force(orc):
    for w in _tiny_cases()[:2]:
        kmin, kmax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, w.block_size)
        bmin, bmax = _brute_meta(w)
        dmin, dmax = _dec(kmin), _dec(kmax)
        for (pb, g, c), v in bmin.items():
            assert dmin[pb, g, c] == v and dmax[pb, g, c] == bmax[(pb, g, c)], (pb, g, c)


def pin_meta_poison_and_step(orc):
    w = workloads.make(1)
    kc = w.key_cache.copy()
    # +-1e4 in the invalid rows of each sequence's last block must not show up.
    for b in range(2):
        L = int(w.context_lens[b])
        pb = int(w.block_tables[b, (L - 1) // 16])
        kc[pb, L % 16 or 16:, :, ::2] = 0x461C      # bf16 10000
        kc[pb, L % 16 or 16:, :, 1::2] = 0xC61C     # bf16 -10000
    kmin, kmax = orc.quest_block_metadata(kc, w.block_tables, w.context_lens, 16)
    assert np.abs(_dec(kmin)).max() < 1e4 and np.abs(_dec(kmax)).max() < 1e4
    # step mode writes only each sequence's last block.
    base = np.full_like(kmin, 0x1234)
    smin, smax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16,
                                          last_block_only=True, key_min=base, key_max=base)
    fmin, fmax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    last = {int(w.block_tables[0, 2]), int(w.block_tables[1, 4])}
    for pb in range(16):
        if pb in last:
            assert np.array_equal(smin[pb], fmin[pb]) and np.array_equal(smax[pb], fmax[pb])
        else:
            assert (smin[pb] == 0x1234).all() and (smax[pb] == 0x1234).all()


# ---------------------------------------------------------------------------
# Quest score and Top-K
# ---------------------------------------------------------------------------

def _frac_score(w, kmin, kmax, b, g, lb):
    G = w.group
    pb = int(w.block_tables[b, lb])
    tot = Fraction(0)
    for h in range(g * G, (g + 1) * G):
        q = _dec(w.query[b, h])
        lo = _dec(kmin[pb, g])
        hi = _dec(kmax[pb, g])
        for c in range(w.head_dim):
            tot += max(Fraction(q[c]) * Fraction(lo[c]), Fraction(q[c]) * Fraction(hi[c]))
    return tot


def pin_score_exact_rational(orc):
    w = workloads.make(1)
    kmin, kmax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    for b in range(2):
        s = orc.quest_block_scores(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, b, 0)
        nb = -(-int(w.context_lens[b]) // 16)
        assert s.size == nb
        for lb in range(nb):
            assert s[lb] == float(_frac_score(w, kmin, kmax, b, 0, lb)), (b, lb)


def pin_score_upper_bound_and_single_token(orc):
    w = workloads.random_case(41, batch=2, num_q_heads=6, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[33, 48])   # seq 0: last block has 1 token
    kmin, kmax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    G = 3
    for b in range(2):
        L = int(w.context_lens[b])
        for g in range(2):
            s = orc.quest_block_scores(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, b, g)
            for lb in range(-(-L // 16)):
                pb = int(w.block_tables[b, lb])
                n = min(16, L - lb * 16)
                dots = []
                for t in range(n):
                    k = _dec(w.key_cache[pb, t, g])
                    dots.append(sum(Fraction(float(x)) * Fraction(float(y))
                                    for h in range(g * G, (g + 1) * G)
                                    for x, y in zip(_dec(w.query[b, h]), k)))
                assert Fraction(float(s[lb])) >= max(dots) - Fraction(1, 10**9), "upper bound"
                if n == 1:
                    assert s[lb] == float(dots[0]), "single-token block score = sum_h q.k"


def _rank_select(scores, k):
    """Independent Top-K: a block is kept iff fewer than k blocks beat it
    (higher score, or equal score and lower index)."""
    n = len(scores)
    keep = []
    for i in range(n):
        beat = sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if beat < k:
            keep.append(i)
    return keep


def pin_topk_rank_and_all(orc):
    w = workloads.random_case(42, batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[100, 16, 77])
    kmin, kmax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    for K in (1, 3, 7, 20):
        sel = orc.quest_select_topk(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, K)
        assert sel.shape == (3, 2, K) and sel.dtype == np.int32
        for b in range(3):
            nb = -(-int(w.context_lens[b]) // 16)
            for g in range(2):
                s = orc.quest_block_scores(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, b, g)
                exp = _rank_select(s.tolist(), K)
                row = sel[b, g].tolist()
                assert row[:len(exp)] == exp and all(x == -1 for x in row[len(exp):]), (K, b, g)
                if K >= nb:
                    assert exp == list(range(nb))


def pin_topk_tie_lower_index(orc):
    """Copy block A's rows into a later block B: equal metadata, equal score.
    With room for one of the two, the lower logical index wins."""
    w = workloads.random_case(43, batch=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
                              block_size=16, context_lens=[64])
    kmin, kmax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    s = orc.quest_block_scores(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, 0, 0)
    best = int(np.argmax(s))
    kc = w.key_cache.copy()
    others = [lb for lb in range(4) if lb != best]
    later = max(others)
    kc[int(w.block_tables[0, later])] = kc[int(w.block_tables[0, best])]
    a, c = min(best, later), max(best, later)
    kmin, kmax = orc.quest_block_metadata(kc, w.block_tables, w.context_lens, 16)
    s2 = orc.quest_block_scores(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, 0, 0)
    assert s2[a] == s2[c]
    sel = orc.quest_select_topk(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, 1)
    assert sel[0, 0, 0] == a, "tie goes to the lower logical block"


# ---------------------------------------------------------------------------
# Sparse attention
# ---------------------------------------------------------------------------

def pin_sparse_all_equals_dense(orc):
    for w in _tiny_cases():
        nbmax = int(w.nblocks().max())
        sel = np.full((w.batch, w.num_kv_heads, nbmax + 2), -1, np.int32)
        for b, nb in enumerate(w.nblocks().tolist()):
            sel[b, :, :nb] = np.arange(nb)
        d = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                       w.context_lens, w.scale)
        s = orc.sparse_paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                              w.context_lens, sel, w.scale)
        assert np.abs(d - s).max() <= TOL


def pin_sparse_equals_dense_on_dropped_context(orc):
    """Sparse attention == dense attention on a table that lists only the selected
    blocks (ascending, so a partial last block stays last)."""
    w = workloads.random_case(51, batch=2, num_q_heads=3, num_kv_heads=1, head_dim=64,
                              block_size=16, context_lens=[90, 64])
    sel = np.array([[[0, 2, 5, -1]], [[1, 3, -1, -1]]], np.int32)
    s = orc.sparse_paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                          w.context_lens, sel, w.scale)
    bt2 = np.full_like(w.block_tables, -1)
    ctx2 = np.zeros(2, np.int32)
    for b in range(2):
        ids = [x for x in sel[b, 0].tolist() if x >= 0]
        bt2[b, :len(ids)] = w.block_tables[b, ids]
        L = int(w.context_lens[b])
        ctx2[b] = sum(min(16, L - lb * 16) for lb in ids)
    d = orc.paged_attention_decode(w.query, w.key_cache, w.value_cache, bt2, ctx2, w.scale)
    assert np.abs(d - s).max() <= TOL


def pin_sparse_brute_force(orc):
    w = workloads.random_case(52, batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[70, 35])
    sel = np.array([[[4, 1, -1], [0, 2, 3]], [[2, -1, -1], [1, 0, -1]]], np.int32)
    s = orc.sparse_paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                          w.context_lens, sel, w.scale)
    for b in range(2):
        L = int(w.context_lens[b])
        for h in range(4):
            g = h // 2
            ids = sorted(x for x in sel[b, g].tolist() if x >= 0)
            pos = [t for lb in ids for t in range(lb * 16, min(lb * 16 + 16, L))]
            q = _dec(w.query[b, h])
            k = np.stack([_dec(w.key_cache[int(w.block_tables[b, t // 16]), t % 16, g]) for t in pos])
            v = np.stack([_dec(w.value_cache[int(w.block_tables[b, t // 16]), t % 16, g]) for t in pos])
            ref = np.array(_ref_row(q, k, v, float(w.scale)))
            assert np.abs(s[b, h] - ref).max() <= TOL, (b, h)


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) KV cache
# ---------------------------------------------------------------------------

def _torch_e4m3(values_f32):
    """torch's CPU float8_e4m3fn conversion (round to nearest even), as codes."""
    import torch
    t = torch.from_numpy(np.asarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_fp8_decode_matches_torch(orc):
    import torch
    c = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_to_f64(c)
    exp = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(exp))
    ok = ~np.isnan(exp)
    assert np.array_equal(got[ok], exp[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(exp[ok]))


def pin_fp8_encode_matches_torch_in_range(orc):
    """Every finite bf16 value of magnitude <= 448 encodes as torch encodes it."""
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    assert np.array_equal(orc.e4m3_from_f32(v), _torch_e4m3(v))


def pin_fp8_encode_saturates_nan_and_sign(orc):
    big = np.array([448.5, 463.9, 464.0, 470.0, 1e4, 3e38, np.inf], np.float32)
    assert (orc.e4m3_from_f32(big) == 0x7E).all()
    assert (orc.e4m3_from_f32(-big) == 0xFE).all()
    assert orc.e4m3_from_f32(np.array([np.nan], np.float32))[0] == 0x7F
    assert orc.e4m3_from_f32(np.array([-0.0], np.float32))[0] == 0x80
    assert orc.e4m3_from_f32(np.array([-1e-30], np.float32))[0] == 0x80


def _e4m3_value_py(code):
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    v = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if s else v


def pin_fp8_encode_nearest_bruteforce(orc):
    """The code of y is a nearest finite value (exact rational distances); on an
    exact tie, the even code."""
    rng = np.random.default_rng(71)
    mags = np.exp2(rng.uniform(-13.0, 9.0, size=400)).astype(np.float32)
    ys = np.concatenate([mags, -mags, np.array([2.0 ** -10, 1.0625, 1.1875, 3 * 2.0 ** -11,
                                                 0.0, 432.0, 240.0], np.float32)])
    finite = [c for c in range(256) if not ((c >> 3) & 15 == 15 and c & 7 == 7)]
    vals = {c: _e4m3_value_py(c) for c in finite}
    codes = orc.e4m3_from_f32(ys)
    for y, c in zip(ys.tolist(), codes.tolist()):
        fy = Fraction(y)
        best = min(abs(v - fy) for v in vals.values())
        assert abs(vals[c] - fy) == best, (y, hex(c))
        ties = [k for k, v in vals.items() if abs(v - fy) == best and (v != 0 or k in (0, 0x80))]
        ties = sorted({k & 0x7F for k in ties})
        if len(ties) > 1:
            assert (c & 0x7F) % 2 == 0, (y, hex(c))


def pin_fp8_quantize_hand_worked(orc):
    """x = 1.0 with scale 3: float32(1/3) * 1.0 = 0.33333334; the E4M3 neighbours
    are 0.3125 (0x2A) and 0.34375 (0x2B); the nearer is 0x2B. With scale 0.5 the
    product is 2.0 exactly: code 0x40."""
    one = np.array([[[0x3F80]]], np.uint16)                 # bf16 1.0, [1, 1, 1]
    assert orc.quantize_fp8(one, [3.0])[0, 0, 0] == 0x2B
    assert orc.quantize_fp8(one, [0.5])[0, 0, 0] == 0x40
    neg = np.array([[[0xC0A0]]], np.uint16)                 # bf16 -5.0
    assert orc.quantize_fp8(neg, [0.5])[0, 0, 0] == 0xD2    # -10 = -(1.25 * 2^3)


def _representable_case(seed, scales):
    """A small paged case whose K/V values are E4M3 values times a power-of-two scale
    per KV head (exact in bf16 and exact under quantisation)."""
    w = workloads.random_case(seed, batch=3, num_q_heads=6, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[1, 40, 70])
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(255) if c not in (0x7F,)], np.uint8)

    def pick(shape):
        codes = rng.choice(finite, size=shape)
        vals = np.asarray(_e4m3_f64_ref(codes)) * np.asarray(scales)[:, None]
        return (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w.key_cache = pick(w.key_cache.shape)
    w.value_cache = pick(w.value_cache.shape)
    return w


def _e4m3_f64_ref(codes):
    return np.vectorize(lambda c: float(_e4m3_value_py(int(c))))(codes)


def pin_fp8_write_roundtrip_exact(orc):
    scales = [0.5, 4.0]
    w = _representable_case(72, scales)
    NB, bs, Hkv, D = w.key_cache.shape
    slots = np.array([3, 40, -1, 17], np.int64)
    rows = w.key_cache[slots[slots >= 0] // bs, slots[slots >= 0] % bs]   # representable rows
    key = np.concatenate([rows, rows[:1]])
    kc0 = np.zeros((NB, bs, Hkv, D), np.uint8)
    kc, vc = orc.reshape_and_cache_fp8(kc0, kc0, key, key, slots, bs, scales, scales)
    back = orc.e4m3_to_f64(kc) * np.asarray(scales)[None, None, :, None]
    for i, s_ in enumerate(slots.tolist()):
        if s_ < 0:
            continue
        assert np.array_equal(back[s_ // bs, s_ % bs], _dec(key[i]))
    written = np.zeros((NB, bs), bool)
    written[slots[slots >= 0] // bs, slots[slots >= 0] % bs] = True
    assert (kc[~written] == 0).all() and np.array_equal(kc, vc)


def pin_fp8_attention_equals_bf16_on_representable(orc):
    """With values exactly representable, FP8 attention is bf16 attention."""
    scales_k, scales_v = [0.5, 4.0], [2.0, 0.25]
    w = _representable_case(73, scales_k)
    wv = _representable_case(74, scales_v)
    vcache = wv.value_cache
    kq = orc.quantize_fp8(w.key_cache, scales_k)
    vq = orc.quantize_fp8(vcache, scales_v)
    got = orc.paged_attention_decode_fp8(w.query, kq, vq, scales_k, scales_v, w.block_tables,
                                         w.context_lens, w.scale)
    exp = orc.paged_attention_decode(w.query, w.key_cache, vcache, w.block_tables,
                                     w.context_lens, w.scale)
    assert np.abs(got - exp).max() <= TOL


def pin_fp8_sparse_all_blocks_equals_fp8_dense(orc):
    """Selecting every block of every KV head is dense FP8 attention."""
    scales_k, scales_v = [0.03, 0.07], [0.05, 0.011]
    w = workloads.random_case(75, batch=3, num_q_heads=6, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[1, 40, 70])
    kq = orc.quantize_fp8(w.key_cache, scales_k)
    vq = orc.quantize_fp8(w.value_cache, scales_v)
    nb = -(-w.context_lens // 16)
    sel = np.full((3, 2, 6), -1, np.int32)
    for b in range(3):
        sel[b, :, :nb[b]] = np.arange(nb[b])[::-1]          # unsorted: order is irrelevant
    got = orc.sparse_paged_attention_decode_fp8(w.query, kq, vq, scales_k, scales_v,
                                                w.block_tables, w.context_lens, sel, w.scale)
    exp = orc.paged_attention_decode_fp8(w.query, kq, vq, scales_k, scales_v, w.block_tables,
                                         w.context_lens, w.scale)
    assert np.abs(got - exp).max() <= TOL


def pin_fp8_sparse_equals_bf16_sparse_on_representable(orc):
    """With exactly representable values and per-head K and V scales that differ, FP8
    sparse attention is bf16 sparse attention, holes and unsorted ids included."""
    scales_k, scales_v = [0.5, 4.0], [2.0, 0.25]
    w = _representable_case(76, scales_k)
    vcache = _representable_case(77, scales_v).value_cache
    kq = orc.quantize_fp8(w.key_cache, scales_k)
    vq = orc.quantize_fp8(vcache, scales_v)
    sel = np.full((3, 2, 4), -1, np.int32)
    sel[0, 0, 0] = 0
    sel[1, 0] = [2, -1, 0, -1]
    sel[1, 1] = [-1, 1, -1, -1]
    sel[2, 0] = [4, 1, -1, 3]
    sel[2, 1] = [0, -1, 2, -1]
    got = orc.sparse_paged_attention_decode_fp8(w.query, kq, vq, scales_k, scales_v,
                                                w.block_tables, w.context_lens, sel, w.scale)
    exp = orc.sparse_paged_attention_decode(w.query, w.key_cache, vcache, w.block_tables,
                                            w.context_lens, sel, w.scale)
    assert np.abs(got - exp).max() <= TOL
    assert (got[0, 3:] == 0).all(), "KV head 1 of sequence 0 selects nothing: zero rows"


# ---------------------------------------------------------------------------
# Quest over E4M3 caches
# ---------------------------------------------------------------------------

def _fp8_code_case(seed):
    """Random finite E4M3 codes (both zeros included) in a paged key cache; the rows
    past each sequence's context hold +-448, which the metadata must not see."""
    w = workloads.random_case(seed, batch=3, num_q_heads=6, num_kv_heads=2, head_dim=64,
                              block_size=16, context_lens=[1, 40, 70])
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    kc = rng.choice(finite, size=w.key_cache.shape).astype(np.uint8)
    for b in range(3):
        L = int(w.context_lens[b])
        pb = int(w.block_tables[b, (L - 1) // 16])
        kc[pb, L % 16 or 16:, :, ::2] = 0x7E       # +448
        kc[pb, L % 16 or 16:, :, 1::2] = 0xFE      # -448
    return w, kc


def pin_fp8_meta_brute_force(orc):
    """Per channel, the decoded codes are the smallest and largest code value over the
    block's valid rows, from a decoder written from the E4M3 definition; step mode
    writes only each sequence's last block."""
    w, kc = _fp8_code_case(81)
    kmin, kmax = orc.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, 16)
    assert kmin.dtype == np.uint8 and kmin.shape == (w.num_blocks, 2, 64)
    val = {c: _e4m3_value_py(c) for c in range(256) if c not in (0x7F, 0xFF)}
    for b in range(3):
        L = int(w.context_lens[b])
        for lb in range(-(-L // 16)):
            pb = int(w.block_tables[b, lb])
            n = min(16, L - lb * 16)
            for g in range(2):
                for c in range(64):
                    vals = [val[int(kc[pb, t, g, c])] for t in range(n)]
                    assert val[int(kmin[pb, g, c])] == min(vals), (pb, g, c)
                    assert val[int(kmax[pb, g, c])] == max(vals), (pb, g, c)
    base = np.full_like(kmin, 0x35)
    smin, smax = orc.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, 16,
                                              last_block_only=True, key_min=base, key_max=base)
    last = {int(w.block_tables[b, (int(w.context_lens[b]) - 1) // 16]) for b in range(3)}
    for pb in range(w.num_blocks):
        if pb in last:
            assert np.array_equal(smin[pb], kmin[pb]) and np.array_equal(smax[pb], kmax[pb])
        else:
            assert (smin[pb] == 0x35).all() and (smax[pb] == 0x35).all()


def pin_fp8_scores_exact_rational(orc):
    """Each FP8 block score is the exact rational bound on the decoded codes, rounded once."""
    w, kc = _fp8_code_case(82)
    kmin, kmax = orc.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, 16)
    G = w.group
    for b in range(3):
        nb = -(-int(w.context_lens[b]) // 16)
        for g in range(2):
            s = orc.quest_block_scores_fp8(w.query, kmin, kmax, w.block_tables, w.context_lens,
                                           16, b, g)
            assert s.size == nb
            for lb in range(nb):
                pb = int(w.block_tables[b, lb])
                tot = Fraction(0)
                for h in range(g * G, (g + 1) * G):
                    q = _dec(w.query[b, h])
                    for c in range(64):
                        qc = Fraction(float(q[c]))
                        tot += max(qc * _e4m3_value_py(int(kmin[pb, g, c])),
                                   qc * _e4m3_value_py(int(kmax[pb, g, c])))
                assert s[lb] == float(tot), (b, g, lb)


def pin_fp8_quest_is_bf16_quest_over_the_scale(orc):
    """On keys that are E4M3 values times a power-of-two scale per KV head, quantising
    commutes with the per-channel min and max, so the FP8 scores are the bf16 scores
    divided by the head's scale (exactly) and both select the same blocks, ties
    included; the selection is the rank rule on the FP8 scores."""
    scales = [0.5, 4.0]
    w = _representable_case(83, scales)
    kq = orc.quantize_fp8(w.key_cache, scales)
    fmin, fmax = orc.quest_block_metadata_fp8(kq, w.block_tables, w.context_lens, 16)
    bmin, bmax = orc.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens, 16)
    for g in range(2):
        assert np.array_equal(_e4m3_f64_ref(fmin[:, g]) * scales[g], _dec(bmin[:, g]))
        assert np.array_equal(_e4m3_f64_ref(fmax[:, g]) * scales[g], _dec(bmax[:, g]))
    for b in range(3):
        for g in range(2):
            sf = orc.quest_block_scores_fp8(w.query, fmin, fmax, w.block_tables, w.context_lens,
                                            16, b, g)
            sb = orc.quest_block_scores(w.query, bmin, bmax, w.block_tables, w.context_lens,
                                        16, b, g)
            assert np.array_equal(sf * scales[g], sb), (b, g)
    for K in (1, 2, 4, 6):
        sel = orc.quest_select_topk_fp8(w.query, fmin, fmax, w.block_tables, w.context_lens, 16, K)
        ref = orc.quest_select_topk(w.query, bmin, bmax, w.block_tables, w.context_lens, 16, K)
        assert sel.shape == (3, 2, K) and sel.dtype == np.int32 and np.array_equal(sel, ref), K
        for b in range(3):
            for g in range(2):
                s = orc.quest_block_scores_fp8(w.query, fmin, fmax, w.block_tables,
                                               w.context_lens, 16, b, g)
                exp = _rank_select(s.tolist(), K)
                row = sel[b, g].tolist()
                assert row[:len(exp)] == exp and all(x == -1 for x in row[len(exp):])


def pin_fp8_topk_tie_lower_index(orc):
    """Two blocks with the same codes tie; with room for one the lower index wins."""
    w, kc = _fp8_code_case(84)
    kmin, kmax = orc.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, 16)
    s = orc.quest_block_scores_fp8(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, 2, 1)
    best = int(np.argmax(s[:4]))                    # full blocks only: no poisoned rows
    later = max(lb for lb in range(4) if lb != best)
    kc[int(w.block_tables[2, later])] = kc[int(w.block_tables[2, best])]
    kmin, kmax = orc.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens, 16)
    s2 = orc.quest_block_scores_fp8(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, 2, 1)
    a, c = min(best, later), max(best, later)
    assert s2[a] == s2[c] and s2[a] == s2.max()
    sel = orc.quest_select_topk_fp8(w.query, kmin, kmax, w.block_tables, w.context_lens, 16, 1)
    assert sel[2, 1, 0] == a, "tie goes to the lower logical block"


# ---------------------------------------------------------------------------
# Multi-token queries (varlen, right-aligned causal mask)
# ---------------------------------------------------------------------------

def pin_varlen_single_token_is_decode(orc):
    """One query token per sequence: the causal limit is the whole context."""
    for w in _tiny_cases():
        w2 = workloads.varlen_case(81, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                                   head_dim=w.head_dim, block_size=w.block_size,
                                   context_lens=w.context_lens, q_lens=[1] * w.batch)
        got = orc.paged_attention_varlen(w2.query_varlen, w2.key_cache, w2.value_cache,
                                         w2.block_tables, w2.context_lens, w2.cu_seqlens_q,
                                         w2.scale)
        exp = orc.paged_attention_decode(w2.query_varlen, w2.key_cache, w2.value_cache,
                                         w2.block_tables, w2.context_lens, w2.scale)
        assert np.abs(got - exp).max() <= TOL


def pin_varlen_torch_sdpa_bottom_right_mask(orc):
    """torch's float64 scaled_dot_product_attention with an explicit boolean mask
    that lets row j see the first ctx - q_len + j + 1 positions, GQA enabled."""
    import torch
    w = workloads.varlen_case(82, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                              context_lens=[37, 80, 16, 5], q_lens=[4, 16, 1, 5])
    got = orc.paged_attention_varlen(w.query_varlen, w.key_cache, w.value_cache, w.block_tables,
                                     w.context_lens, w.cu_seqlens_q, w.scale)
    cu = w.cu_seqlens_q
    for b, L in enumerate(w.context_lens.tolist()):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        n = r1 - r0
        rows = [int(x) for x in w.block_tables[b, :-(-L // 16)]]
        k = np.concatenate([_dec(w.key_cache[p_]) for p_ in rows])[:L]     # [L, Hkv, D]
        v = np.concatenate([_dec(w.value_cache[p_]) for p_ in rows])[:L]
        q = _dec(w.query_varlen[r0:r1])                                      # [n, Hq, D]
        mask = np.zeros((n, L), bool)
        for j in range(n):
            mask[j, :max(0, L - n + j + 1)] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
            torch.from_numpy(v).permute(1, 0, 2)[None], attn_mask=torch.from_numpy(mask),
            scale=float(np.float32(w.scale)), enable_gqa=True)[0].permute(1, 0, 2).numpy()
        ok = mask.any(axis=1)
        assert np.abs(got[r0:r1][ok] - ref[ok]).max() <= TOL
        assert (got[r0:r1][~ok] == 0).all()


def pin_varlen_brute_force_and_short_context(orc):
    """Pure-Python loops with math.fsum; one sequence has more query rows than
    positions, so its first rows see nothing (zero rows)."""
    w = workloads.varlen_case(83, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                              context_lens=[3, 20], q_lens=[5, 6])
    got = orc.paged_attention_varlen(w.query_varlen, w.key_cache, w.value_cache, w.block_tables,
                                     w.context_lens, w.cu_seqlens_q, w.scale)
    sc = float(np.float32(w.scale))
    cu = w.cu_seqlens_q
    for b, L in enumerate(w.context_lens.tolist()):
        n = int(cu[b + 1] - cu[b])
        for j in range(n):
            r = int(cu[b]) + j
            vis = [t for t in range(L) if t <= L - n + j]
            for h in range(4):
                g = h // 2
                qv = _dec(w.query_varlen[r, h]).tolist()
                if not vis:
                    assert (got[r, h] == 0).all()
                    continue
                sc_ = []
                for t in vis:
                    pb = int(w.block_tables[b, t // 16])
                    kv = _dec(w.key_cache[pb, t % 16, g]).tolist()
                    sc_.append(sc * math.fsum(a * c for a, c in zip(qv, kv)))
                m = max(sc_)
                e = [math.exp(x - m) for x in sc_]
                den = math.fsum(e)
                for d in range(64):
                    num = math.fsum(e[i] * float(_dec(w.value_cache[int(w.block_tables[b, t // 16]),
                                                                    t % 16, g, d]))
                                    for i, t in enumerate(vis))
                    assert abs(num / den - got[r, h, d]) <= TOL


def pin_varlen_mask_edge(orc):
    """Row j of a 6-token chunk over 40 positions sees positions 0 .. 34 + j: changing
    K/V at 35 + j leaves it unchanged, changing 34 + j moves it."""
    w = workloads.varlen_case(84, num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=16,
                              context_lens=[40], q_lens=[6])
    base = orc.paged_attention_varlen(w.query_varlen, w.key_cache, w.value_cache, w.block_tables,
                                      w.context_lens, w.cu_seqlens_q, w.scale)
    for j in (0, 2, 4):
        for t, moves in ((35 + j, False), (34 + j, True)):
            kc, vc = w.key_cache.copy(), w.value_cache.copy()
            pb = int(w.block_tables[0, t // 16])
            kc[pb, t % 16] ^= np.uint16(0x0040)
            vc[pb, t % 16] ^= np.uint16(0x0040)
            out = orc.paged_attention_varlen(w.query_varlen, kc, vc, w.block_tables,
                                             w.context_lens, w.cu_seqlens_q, w.scale)
            changed = np.abs(out[j] - base[j]).max() > 0
            assert changed == moves, (j, t)


# ---------------------------------------------------------------------------
# Multi-token queries over E4M3 caches
# ---------------------------------------------------------------------------

def pin_varlen_fp8_single_token_is_fp8_decode(orc):
    """One query token per sequence over quantised caches: the FP8 decode result."""
    w = workloads.varlen_case(85, num_q_heads=6, num_kv_heads=2, head_dim=64, block_size=16,
                              context_lens=[1, 40, 70], q_lens=[1, 1, 1])
    ks, vs = [0.031, 0.2], [0.5, 0.0123]
    kq = orc.quantize_fp8(w.key_cache, ks)
    vq = orc.quantize_fp8(w.value_cache, vs)
    got = orc.paged_attention_varlen_fp8(w.query_varlen, kq, vq, ks, vs, w.block_tables,
                                         w.context_lens, w.cu_seqlens_q, w.scale)
    exp = orc.paged_attention_decode_fp8(w.query_varlen, kq, vq, ks, vs, w.block_tables,
                                         w.context_lens, w.scale)
    assert np.abs(got - exp).max() <= TOL


def pin_varlen_fp8_equals_bf16_on_representable(orc):
    """With values exactly representable, FP8 varlen attention is bf16 varlen attention
    (chunks longer than the context included)."""
    scales_k, scales_v = [0.5, 4.0], [2.0, 0.25]
    w = _representable_case(86, scales_k)
    wv = _representable_case(87, scales_v)
    wq = workloads.varlen_case(88, num_q_heads=6, num_kv_heads=2, head_dim=64, block_size=16,
                               context_lens=w.context_lens.tolist(), q_lens=[3, 17, 40])
    kq = orc.quantize_fp8(w.key_cache, scales_k)
    vq = orc.quantize_fp8(wv.value_cache, scales_v)
    got = orc.paged_attention_varlen_fp8(wq.query_varlen, kq, vq, scales_k, scales_v,
                                         w.block_tables, w.context_lens, wq.cu_seqlens_q, w.scale)
    exp = orc.paged_attention_varlen(wq.query_varlen, w.key_cache, wv.value_cache, w.block_tables,
                                     w.context_lens, wq.cu_seqlens_q, w.scale)
    assert np.abs(got - exp).max() <= TOL
    assert (got[0] == 0).all() and (got[1] == 0).all()   # 3 rows over 1 position: two see nothing


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
