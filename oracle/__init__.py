"""CPU oracle for paged GQA decode attention, its write path and Quest.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this package: only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code with the HIP library or its Python
binding and imports neither.

Plain numpy, float64 throughout. bf16 inputs arrive as raw uint16 bit patterns
and are decoded exactly (bf16 -> f32 is a 16-bit shift; f32 -> f64 is exact), so
the oracle sees the very values the GPU sees.

Where the method has a closed definition (a cache write, softmax attention over a
token set, a min/max over a block) the oracle is that definition written out; the
online-softmax and split-KV machinery that a kernel uses to reach the same result
appear here only in ``split_kv_partials`` / ``split_kv_combine``, which exist to pin
the combine formula. Quest is a heuristic, so its scoring and Top-K follow the
steps in order.

Sources (page title, section):
  [ASC]  "Ascend Kernel-to-Serving Pipeline" -- sections "ReshapeAndCache",
         "GQA Paged Attention", "Quest Sparse Attention", "Sparse precision".
  [TL18] TileLang tutorial ch. 18 (end-to-end inference serving) -- sections 2.4
         (KV cache structure), 2.6 (paged KV), 4.1 (decode attention / split-KV).

Readings where the pages are silent:
  R1 cache layout [NB, block_size, H_kv, D] for K and V ([TL18] 2.6).
  R2 query head h uses KV head h // (H_q / H_kv) (contiguous groups).
  R3 scores are scale * q.k with scale passed in (1/sqrt(D) in every workload).
  R4 ctx_b = 0 gives a zero output row.
  R5 Quest block score = sum over the group's query heads and channels of
     max(q*kmin, q*kmax); ties in Top-K go to the lower logical block; selected ids
     ascending, padded with -1; K >= nb selects every block.
  R6 masked / unselected tokens contribute exactly nothing (even if their K/V
     bits are NaN).
  R8 multi-token queries ([TL18] 2.7 varlen batches, 3.3 item 4): the query rows of
     sequence b are its newest q_len_b positions, already in the cache; row j
     (0-based) sees positions t <= ctx_b - q_len_b + j (a causal mask aligned to
     the right); a row that sees no position gets a zero output.
  R9 Quest over E4M3 caches: the metadata holds the codes of each channel's
     smallest and largest key code value over a block's valid rows (one byte per
     channel; the keys are code * k_scale[g] with a positive per-head scale, so
     their extremes are the scale times these); the block score is the R5 bound
     on the code values, the scale left out: it multiplies every score of a KV
     head by the same positive factor, and only the order within a head is used.
  R7 FP8 KV cache (the KV-quantisation lever of [TL18] 2.5 and 3.1): codes are
     OCP FP8 E4M3 (bias 7, no infinities, largest finite 448); K and V each carry
     one float32 scale per KV head. Stored code = the E4M3 value nearest to
     float32(x) * float32(1 / scale) (both float32 operations), ties to the even
     code, magnitudes past 448 saturating to 448, NaN to 0x7F; the value read back
     is code * scale.

Parity pins for every function live in tests/test_oracle.py; none of them
re-types a formula from here.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16_exact", "reshape_and_cache", "gather_sequence",
    "paged_attention_decode", "quest_block_metadata", "quest_block_scores",
    "quest_select_topk", "sparse_token_positions", "sparse_paged_attention_decode",
    "split_kv_partials", "split_kv_combine", "e4m3_to_f64", "e4m3_from_f32",
    "fp8_inverse_scale", "quantize_fp8", "reshape_and_cache_fp8", "paged_attention_decode_fp8",
    "sparse_paged_attention_decode_fp8",
    "paged_attention_varlen", "paged_attention_varlen_fp8",
    "e4m3_code_of", "quest_block_metadata_fp8", "quest_block_scores_fp8", "quest_select_topk_fp8",
]


# ---------------------------------------------------------------------------
# bf16 bit patterns <-> float64 (exact)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode: a bf16 pattern is the top half of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Encode values that are already bf16-representable (min/max results)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    if np.any((u & np.uint32(0xFFFF)) != 0):
        raise ValueError("value is not exactly representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# C1 -- ReshapeAndCache  ([ASC] "ReshapeAndCache")
# ---------------------------------------------------------------------------

def reshape_and_cache(key_cache, value_cache, key, value, slot_mapping, block_size):
    """Scatter each new token's K and V row into the paged cache.

    For token i with slot s = slot_mapping[i]: s < 0 means skip; otherwise the
    physical block is s // block_size and the row inside it is s % block_size.
    Returns new (key_cache, value_cache) arrays; the inputs are not modified.
    Bit copies: the uint16 patterns move unchanged.
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    num_blocks = kc.shape[0]
    seen = set()
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64).tolist()):
        if s < 0:
            continue
        if s >= num_blocks * block_size:
            raise ValueError(f"slot {s} outside the cache (precondition)")
        if s in seen:
            raise ValueError(f"slot {s} written twice (precondition)")
        seen.add(s)
        blk, off = divmod(s, block_size)
        kc[blk, off] = key[i]
        vc[blk, off] = value[i]
    return kc, vc


# ---------------------------------------------------------------------------
# C2 -- dense GQA paged decode attention  ([ASC] "GQA Paged Attention"; [TL18] 2.6)
# ---------------------------------------------------------------------------

def _check_table(block_tables, context_lens, block_size, num_blocks):
    for b, L in enumerate(np.asarray(context_lens).tolist()):
        if L < 0:
            raise ValueError("negative context length")
        nb = -(-L // block_size)
        ids = np.asarray(block_tables[b, :nb], dtype=np.int64)
        if ids.size and (ids.min() < 0 or ids.max() >= num_blocks):
            raise ValueError(f"block id out of range in sequence {b} (precondition)")


def gather_sequence(cache_f64, block_tables, b, positions, block_size):
    """Rows of logical positions ``positions`` of sequence b: [n, H_kv, D]."""
    pos = np.asarray(positions, dtype=np.int64)
    pb = np.asarray(block_tables[b], dtype=np.int64)[pos // block_size]
    return cache_f64[pb, pos % block_size]


def _softmax_attention(q, k, v, scale):
    """Softmax attention of one query row set over a token set, by definition.

    q: [G, D]; k, v: [n, D]. p_t = exp(s_t) / sum_u exp(s_u) with s = scale * q.k;
    the max is subtracted only to keep exp in range (it cancels exactly in math).
    """
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    s = scale * (q @ k.T)                       # [G, n]
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v


def paged_attention_decode(query, key_cache, value_cache, block_tables, context_lens,
                           scale, seqs=None):
    """out[b, h, :] = softmax_t(scale * q[b,h].K_t) . V_t over t < ctx_b.

    Token t of sequence b lives at block_tables[b, t // bs], row t % bs; query head
    h reads KV head h // G. Returns float64 [B, H_q, D] (rows of sequences not in
    ``seqs`` stay zero when a subset is requested).
    """
    B, Hq, D = query.shape
    NB, bs, Hkv, _ = key_cache.shape
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    ctx = np.asarray(context_lens, dtype=np.int64)
    _check_table(block_tables, ctx, bs, NB)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    q = bf16_to_f64(query)
    sc = float(np.float32(scale))
    for b in (range(B) if seqs is None else seqs):
        pos = np.arange(int(ctx[b]))
        k = bf16_to_f64(gather_sequence(key_cache, block_tables, b, pos, bs))
        v = bf16_to_f64(gather_sequence(value_cache, block_tables, b, pos, bs))
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            out[b, heads] = _softmax_attention(q[b, heads], k[:, g], v[:, g], sc)
    return out


# ---------------------------------------------------------------------------
# C6 -- split-KV partials and combine  ([TL18] 4.1; used to pin the combine rule)
# ---------------------------------------------------------------------------

def split_kv_partials(q, k, v, scale, bounds):
    """Per split [lo, hi): normalised partial output O_s and log-sum-exp lse_s.

    q: [G, D]; k, v: [n, D]. Each split keeps its own max m_s, l_s = sum exp(s - m_s),
    O_s = sum exp(s - m_s) v / l_s and lse_s = m_s + ln l_s. An empty split has
    lse = -inf and O_s = 0.
    """
    G, D = q.shape
    outs, lses = [], []
    for lo, hi in bounds:
        if hi <= lo:
            outs.append(np.zeros((G, v.shape[1])))
            lses.append(np.full(G, -np.inf))
            continue
        s = scale * (q @ k[lo:hi].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        outs.append((e @ v[lo:hi]) / l)
        lses.append((m + np.log(l))[:, 0])
    return np.stack(outs), np.stack(lses)


def split_kv_combine(outs, lses):
    """O = sum_s exp(lse_s - LSE) O_s with LSE = ln sum_s exp(lse_s).

    Each split's own normaliser is rescaled to a common reference before weighting
    (the tutorial's l_s / sum l weights, read with every l_s taken relative to one
    shared max). All splits empty -> zeros.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    mx = lses.max(axis=0)                                    # [G]
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lses - safe)                                  # [S, G]; exp(-inf) = 0
    tot = w.sum(axis=0)
    res = np.einsum("sg,sgd->gd", w, outs)
    with np.errstate(invalid="ignore", divide="ignore"):
        res = np.where(tot[:, None] > 0, res / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    return res


# ---------------------------------------------------------------------------
# C3 -- Quest block metadata (per block, per KV head, per channel key min / max)
# ---------------------------------------------------------------------------

def quest_block_metadata(key_cache, block_tables, context_lens, block_size,
                         last_block_only=False, key_min=None, key_max=None):
    """kmin/kmax[pb, g, c] over the *valid* tokens of each referenced block.

    For every sequence b and logical block lb < nb_b (only lb = nb_b - 1 in step
    mode), pb = block_tables[b, lb] and the block holds n = min(bs, ctx_b - lb*bs)
    valid tokens; tokens past the context are skipped ([ASC] Quest requirements).
    Blocks not referenced keep their previous contents (``key_min``/``key_max``
    inputs, zeros if not given). Returns uint16 bf16 patterns [NB, H_kv, D].
    """
    NB, bs, Hkv, D = key_cache.shape
    assert bs == block_size
    kmin = np.zeros((NB, Hkv, D), np.uint16) if key_min is None else np.array(key_min, copy=True)
    kmax = np.zeros((NB, Hkv, D), np.uint16) if key_max is None else np.array(key_max, copy=True)
    ctx = np.asarray(context_lens, dtype=np.int64)
    _check_table(block_tables, ctx, bs, NB)
    for b, L in enumerate(ctx.tolist()):
        nb = -(-L // bs)
        blocks = [nb - 1] if (last_block_only and nb > 0) else range(nb)
        for lb in blocks:
            pb = int(block_tables[b, lb])
            n = min(bs, L - lb * bs)
            k = bf16_to_f64(key_cache[pb, :n])          # [n, H_kv, D]
            kmin[pb] = f64_to_bf16_exact(k.min(axis=0))
            kmax[pb] = f64_to_bf16_exact(k.max(axis=0))
    return kmin, kmax


# ---------------------------------------------------------------------------
# C4 -- Quest score and Top-K selection  ([ASC] "Quest Sparse Attention")
# ---------------------------------------------------------------------------

def quest_block_scores(query, key_min, key_max, block_tables, context_lens, block_size, b, g):
    """Score of every logical block lb < nb_b of sequence b for KV head g.

    score(lb) = sum over query heads h of group g and channels c of
    max(q[b,h,c] * kmin[pb,g,c], q[b,h,c] * kmax[pb,g,c]), pb = block_tables[b, lb]:
    an upper bound of sum_h q_h . k_t over the block's valid tokens. bf16 x bf16
    products are exact in float64; math.fsum returns the correctly rounded sum, so
    each score is the exact real value rounded once.
    """
    Hq = query.shape[1]
    Hkv = key_min.shape[1]
    G = Hq // Hkv
    L = int(context_lens[b])
    nb = -(-L // block_size)
    q = bf16_to_f64(query[b, g * G:(g + 1) * G])             # [G, D]
    pbs = np.asarray(block_tables[b, :nb], dtype=np.int64)
    lo = bf16_to_f64(key_min[pbs, g])                        # [nb, D]
    hi = bf16_to_f64(key_max[pbs, g])
    terms = np.maximum(q[None, :, :] * lo[:, None, :], q[None, :, :] * hi[:, None, :])
    return np.array([math.fsum(t.ravel().tolist()) for t in terms], dtype=np.float64)


def quest_select_topk(query, key_min, key_max, block_tables, context_lens, block_size, topk):
    """[B, H_kv, topk] int32: per (b, g) the min(topk, nb_b) best logical blocks.

    Order by score descending, equal scores by lower logical index; the kept ids
    are returned ascending and padded with -1.
    """
    return _topk_of_scores(
        lambda b, g: quest_block_scores(query, key_min, key_max, block_tables, context_lens,
                                        block_size, b, g),
        query.shape[0], key_min.shape[1], topk)


def _topk_of_scores(scores_of, B, Hkv, topk):
    """The Top-K rule over the scores ``scores_of(b, g)`` of each (sequence, KV head)."""
    if topk < 1:
        raise ValueError("topk_blocks must be >= 1")
    out = np.full((B, Hkv, topk), -1, dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            s = scores_of(b, g)
            order = sorted(range(s.size), key=lambda lb: (-s[lb], lb))
            keep = sorted(order[:min(topk, s.size)])
            out[b, g, :len(keep)] = keep
    return out


# ---------------------------------------------------------------------------
# C5 -- sparse paged attention over the selected blocks  ([ASC] "Quest", "Sparse precision")
# ---------------------------------------------------------------------------

def sparse_token_positions(topk_row, ctx, block_size):
    """Logical positions covered by the selected blocks of one (b, g), t < ctx."""
    ids = sorted({int(x) for x in np.asarray(topk_row).tolist() if x >= 0})
    nb = -(-int(ctx) // block_size)
    pos = []
    for lb in ids:
        if lb >= nb:
            raise ValueError("selected block past the context (precondition)")
        pos.extend(range(lb * block_size, min((lb + 1) * block_size, int(ctx))))
    return np.asarray(pos, dtype=np.int64)


def sparse_paged_attention_decode(query, key_cache, value_cache, block_tables, context_lens,
                                  topk_indices, scale, seqs=None):
    """Exact softmax attention over only the tokens of the selected blocks.

    The selection is per KV head: every query head of group g attends to the
    tokens of topk_indices[b, g] (entries -1 are ignored). With the selection fixed,
    this is C2 restricted to that token set.
    """
    B, Hq, D = query.shape
    NB, bs, Hkv, _ = key_cache.shape
    G = Hq // Hkv
    ctx = np.asarray(context_lens, dtype=np.int64)
    _check_table(block_tables, ctx, bs, NB)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    q = bf16_to_f64(query)
    sc = float(np.float32(scale))
    for b in (range(B) if seqs is None else seqs):
        for g in range(Hkv):
            pos = sparse_token_positions(topk_indices[b, g], ctx[b], bs)
            # rows of KV head g only: [n, D]
            k = bf16_to_f64(gather_sequence(key_cache[:, :, g], block_tables, b, pos, bs))
            v = bf16_to_f64(gather_sequence(value_cache[:, :, g], block_tables, b, pos, bs))
            heads = slice(g * G, (g + 1) * G)
            out[b, heads] = _softmax_attention(q[b, heads], k, v, sc)
    return out


# ---------------------------------------------------------------------------
# C7 -- FP8 (OCP E4M3) KV cache: quantise on write, dequantise on read  (R7)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def _e4m3_closed_form(codes: np.ndarray) -> np.ndarray:
    """Closed-form decode: sign s, exponent e (4 bits, bias 7), mantissa m (3 bits);
    e = 0 is subnormal (m * 2^-9); e = 15 with m = 7 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >= 128, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# The closed form evaluated once for all 256 codes; decoding is then a lookup.
_E4M3_ALL = _e4m3_closed_form(np.arange(256, dtype=np.uint8))


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code (the closed form above, looked up per code)."""
    return _E4M3_ALL[np.asarray(codes, dtype=np.uint8)]


# The finite non-negative values in code order (codes 0x00 .. 0x7E), increasing.
_E4M3_POS = e4m3_to_f64(np.arange(127, dtype=np.uint8))


def e4m3_from_f32(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value to each float32 y (by value), ties to the even code;
    |y| > 448 saturates to 448; NaN gives 0x7F. The sign bit follows y's (so -0
    and negative values that round to zero give 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    a_clip = np.minimum(a, E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a_clip, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = np.abs(a_clip - _E4M3_POS[lo])
    d_hi = np.abs(_E4M3_POS[hi] - a_clip)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = pick.astype(np.uint8) | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def fp8_inverse_scale(scale) -> np.ndarray:
    """float32(1 / scale), one float32 division per KV head."""
    return np.float32(1.0) / np.asarray(scale, dtype=np.float32)


def quantize_fp8(x_bits: np.ndarray, scale) -> np.ndarray:
    """bf16 rows [..., H_kv, D] -> E4M3 codes, per KV head g: e4m3(x * (1/scale_g))."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    inv = fp8_inverse_scale(scale)                      # [H_kv]
    y = (x * inv[:, None]).astype(np.float32)           # one float32 rounding
    return e4m3_from_f32(y)


def reshape_and_cache_fp8(key_cache, value_cache, key, value, slot_mapping, block_size,
                          k_scale, v_scale):
    """ReshapeAndCache into E4M3 caches: the same slot rule as ``reshape_and_cache``,
    each row quantised with its KV head's scale. Returns new (key_cache, value_cache)."""
    kq = quantize_fp8(key, k_scale)
    vq = quantize_fp8(value, v_scale)
    return reshape_and_cache(key_cache, value_cache, kq, vq, slot_mapping, block_size)


def paged_attention_decode_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables,
                               context_lens, scale, seqs=None):
    """Dense decode attention over E4M3 caches: the definition of
    ``paged_attention_decode`` applied to K = code * k_scale[g], V = code * v_scale[g]."""
    B, Hq, D = query.shape
    NB, bs, Hkv, _ = key_cache.shape
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    ctx = np.asarray(context_lens, dtype=np.int64)
    _check_table(block_tables, ctx, bs, NB)
    ks = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
    vs = np.asarray(v_scale, dtype=np.float32).astype(np.float64)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    q = bf16_to_f64(query)
    sc = float(np.float32(scale))
    for b in (range(B) if seqs is None else seqs):
        pos = np.arange(int(ctx[b]))
        k = e4m3_to_f64(gather_sequence(key_cache, block_tables, b, pos, bs)) * ks[:, None]
        v = e4m3_to_f64(gather_sequence(value_cache, block_tables, b, pos, bs)) * vs[:, None]
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            out[b, heads] = _softmax_attention(q[b, heads], k[:, g], v[:, g], sc)
    return out


def sparse_paged_attention_decode_fp8(query, key_cache, value_cache, k_scale, v_scale,
                                      block_tables, context_lens, topk_indices, scale, seqs=None):
    """Quest sparse attention over E4M3 caches: the definition of
    ``sparse_paged_attention_decode`` (softmax over the tokens of the blocks that
    topk_indices[b, g] selects, t < ctx_b) applied to K = code * k_scale[g] and
    V = code * v_scale[g]."""
    B, Hq, D = query.shape
    NB, bs, Hkv, _ = key_cache.shape
    G = Hq // Hkv
    ctx = np.asarray(context_lens, dtype=np.int64)
    _check_table(block_tables, ctx, bs, NB)
    ks = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
    vs = np.asarray(v_scale, dtype=np.float32).astype(np.float64)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    q = bf16_to_f64(query)
    sc = float(np.float32(scale))
    for b in (range(B) if seqs is None else seqs):
        for g in range(Hkv):
            pos = sparse_token_positions(topk_indices[b, g], ctx[b], bs)
            k_g = e4m3_to_f64(gather_sequence(key_cache[:, :, g], block_tables, b, pos, bs)) * ks[g]
            v_g = e4m3_to_f64(gather_sequence(value_cache[:, :, g], block_tables, b, pos, bs)) * vs[g]
            heads = slice(g * G, (g + 1) * G)
            out[b, heads] = _softmax_attention(q[b, heads], k_g, v_g, sc)
    return out


# ---------------------------------------------------------------------------
# C9 -- Quest over E4M3 caches  (R9)
# ---------------------------------------------------------------------------

def e4m3_code_of(values: np.ndarray) -> np.ndarray:
    """The E4M3 code of values that are E4M3 values (exact; -0 gives 0x80)."""
    return e4m3_from_f32(np.asarray(values, dtype=np.float64).astype(np.float32))


def quest_block_metadata_fp8(key_cache, block_tables, context_lens, block_size,
                             last_block_only=False, key_min=None, key_max=None):
    """Quest metadata of an E4M3 key cache: the codes of the smallest and largest key
    code value per (referenced block, KV head, channel) over the block's valid rows,
    as ``quest_block_metadata`` takes them over bf16 keys. uint8 [NB, H_kv, D]."""
    NB, bs, Hkv, D = key_cache.shape
    assert bs == block_size
    kmin = np.zeros((NB, Hkv, D), np.uint8) if key_min is None else np.array(key_min, copy=True)
    kmax = np.zeros((NB, Hkv, D), np.uint8) if key_max is None else np.array(key_max, copy=True)
    ctx = np.asarray(context_lens, dtype=np.int64)
    _check_table(block_tables, ctx, bs, NB)
    for b, L in enumerate(ctx.tolist()):
        nb = -(-L // bs)
        blocks = [nb - 1] if (last_block_only and nb > 0) else range(nb)
        for lb in blocks:
            pb = int(block_tables[b, lb])
            n = min(bs, L - lb * bs)
            k = e4m3_to_f64(key_cache[pb, :n])           # [n, H_kv, D]
            kmin[pb] = e4m3_code_of(k.min(axis=0))
            kmax[pb] = e4m3_code_of(k.max(axis=0))
    return kmin, kmax


def quest_block_scores_fp8(query, key_min, key_max, block_tables, context_lens, block_size,
                           b, g):
    """``quest_block_scores`` over E4M3 metadata: the bound on the key code values.
    bf16 x E4M3 products are exact in float64; math.fsum rounds each sum once."""
    Hq = query.shape[1]
    Hkv = key_min.shape[1]
    G = Hq // Hkv
    L = int(context_lens[b])
    nb = -(-L // block_size)
    q = bf16_to_f64(query[b, g * G:(g + 1) * G])             # [G, D]
    pbs = np.asarray(block_tables[b, :nb], dtype=np.int64)
    lo = e4m3_to_f64(key_min[pbs, g])                        # [nb, D]
    hi = e4m3_to_f64(key_max[pbs, g])
    terms = np.maximum(q[None, :, :] * lo[:, None, :], q[None, :, :] * hi[:, None, :])
    return np.array([math.fsum(t.ravel().tolist()) for t in terms], dtype=np.float64)


def quest_select_topk_fp8(query, key_min, key_max, block_tables, context_lens, block_size, topk):
    """``quest_select_topk`` with the scores of ``quest_block_scores_fp8``."""
    return _topk_of_scores(
        lambda b, g: quest_block_scores_fp8(query, key_min, key_max, block_tables,
                                            context_lens, block_size, b, g),
        query.shape[0], key_min.shape[1], topk)


# ---------------------------------------------------------------------------
# C8 -- multi-token queries over the paged cache  (R8; [TL18] 2.7, 3.3)
# ---------------------------------------------------------------------------

def _varlen_attention(query, cu_seqlens_q, context_lens, kv_of, num_kv_heads, scale, seqs):
    """The definition behind the varlen functions: kv_of(b, positions) gives that
    sequence's K and V values [L, H_kv, D] in float64."""
    UQ, Hq, D = query.shape
    Hkv = num_kv_heads
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    ctx = np.asarray(context_lens, dtype=np.int64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    out = np.zeros((UQ, Hq, D), dtype=np.float64)
    q = bf16_to_f64(query)
    sc = float(np.float32(scale))
    for b in (range(ctx.size) if seqs is None else seqs):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = int(ctx[b])
        if r1 <= r0 or L == 0:
            continue
        pos = np.arange(L)
        k, v = kv_of(b, pos)
        lim = L - (r1 - r0) + np.arange(r1 - r0)          # last visible position per row
        visible = pos[None, :] <= lim[:, None]            # [q_len, L]
        for g in range(Hkv):
            for hl in range(G):
                h = g * G + hl
                s_ = sc * (q[r0:r1, h] @ k[:, g].T)        # [q_len, L]
                s_ = np.where(visible, s_, -np.inf)
                m = s_.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.where(visible, np.exp(s_ - m), 0.0)
                den = e.sum(axis=1, keepdims=True)
                p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
                out[r0:r1, h] = p @ v[:, g]
    return out


def paged_attention_varlen(query, key_cache, value_cache, block_tables, context_lens,
                           cu_seqlens_q, scale, seqs=None):
    """out[r, h, :] for every query row r: row j of sequence b (r = cu[b] + j) is
    softmax_t(scale * q[r,h].K_t) . V_t over positions t <= ctx_b - q_len_b + j, by
    definition (all scores, the masked ones set to -inf, then the softmax).
    query: [sum q_len, H_q, D] bf16 bits; returns float64 of that shape."""
    NB, bs, Hkv, _ = key_cache.shape
    _check_table(block_tables, np.asarray(context_lens, dtype=np.int64), bs, NB)

    def kv_of(b, pos):
        return (bf16_to_f64(gather_sequence(key_cache, block_tables, b, pos, bs)),
                bf16_to_f64(gather_sequence(value_cache, block_tables, b, pos, bs)))
    return _varlen_attention(query, cu_seqlens_q, context_lens, kv_of, Hkv, scale, seqs)


def paged_attention_varlen_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables,
                               context_lens, cu_seqlens_q, scale, seqs=None):
    """paged_attention_varlen over E4M3 caches (R7 with R8): K = code * k_scale[g],
    V = code * v_scale[g]."""
    NB, bs, Hkv, _ = key_cache.shape
    _check_table(block_tables, np.asarray(context_lens, dtype=np.int64), bs, NB)
    ks = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
    vs = np.asarray(v_scale, dtype=np.float32).astype(np.float64)

    def kv_of(b, pos):
        return (e4m3_to_f64(gather_sequence(key_cache, block_tables, b, pos, bs)) * ks[:, None],
                e4m3_to_f64(gather_sequence(value_cache, block_tables, b, pos, bs)) * vs[:, None])
    return _varlen_attention(query, cu_seqlens_q, context_lens, kv_of, Hkv, scale, seqs)
