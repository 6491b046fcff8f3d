"""GPU parity of the FP8 (OCP E4M3) cache path against the CPU oracle.

Bars: cache codes bit-exact; attention within max-abs 2e-3 of the float64 oracle
evaluated on the oracle's own codes (the error of quantising itself is not part of
the bar). On the full-size workloads the GPU quantises the whole pool with its own
write call and the oracle quantises the whole pool independently; the two pools
must agree bit for bit before attention is compared, on every sequence.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import BF, Dev, fp8_codes, max_abs, oracle_selection, to_dev, workload

pytestmark = pytest.mark.gpu
ATOL = 2e-3
U8 = torch.uint8


def _scales(cache_bits, divisor=256.0, stride=7):
    """Per KV head: max |x| over a fixed subsample of the cache, / divisor (so the
    largest values land near 256 of E4M3's 448)."""
    Hkv, D = cache_bits.shape[-2:]
    sub = cache_bits.reshape(-1, Hkv, D)[::stride]
    x = (sub.astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.abs(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0)).max(axis=(0, 2))
    return np.maximum(amax / divisor, 1e-3).astype(np.float32)


def _codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------------------
# Write path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ks,vs", [((0.1, 7.0), (1.0, 0.0625)), ((1.0, 3.0), (250.0, 1e-3))])
def test_fp8_write_every_bf16_value(ks, vs):
    """All 65536 bf16 patterns (NaN, inf, subnormals, both zeros) through the write."""
    Hkv, D, bs, NB = 2, 128, 16, 40
    T = 65536 // (Hkv * D)
    allbits = np.arange(65536, dtype=np.uint16)
    key = allbits.reshape(T, Hkv, D)
    value = allbits[::-1].copy().reshape(T, Hkv, D)
    rng = np.random.default_rng(5)
    slots = rng.permutation(NB * bs)[:T].astype(np.int64)
    slots[[3, 77]] = -1
    zeros = np.zeros((NB, bs, Hkv, D), np.uint8)
    kc, vc = torch.zeros((NB, bs, Hkv, D), dtype=U8, device="cuda"), torch.zeros(
        (NB, bs, Hkv, D), dtype=U8, device="cuda")
    d_ks = torch.tensor(ks, dtype=torch.float32, device="cuda")
    d_vs = torch.tensor(vs, dtype=torch.float32, device="cuda")
    gp.reshape_and_cache_fp8(to_dev(key, BF), to_dev(value, BF), kc, vc, d_ks, d_vs,
                             to_dev(slots, torch.int64))
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache_fp8(zeros, zeros, key, value, slots, bs, ks, vs)
    assert np.array_equal(_codes(kc), ek), "key codes differ from the oracle"
    assert np.array_equal(_codes(vc), ev), "value codes differ from the oracle"


@pytest.mark.parametrize("config", [1, 3])
def test_fp8_write_config(config):
    w = workload(config)
    ks, vs = _scales(w.key_cache), _scales(w.value_cache)
    shape = w.key_cache.shape
    kc = torch.zeros(shape, dtype=U8, device="cuda")
    vc = torch.zeros(shape, dtype=U8, device="cuda")
    gp.reshape_and_cache_fp8(to_dev(w.new_key, BF), to_dev(w.new_value, BF), kc, vc,
                             to_dev(ks, torch.float32), to_dev(vs, torch.float32),
                             to_dev(w.slot_mapping, torch.int64))
    torch.cuda.synchronize()
    s = w.slot_mapping[w.slot_mapping >= 0]
    bs = w.block_size
    z = np.zeros(shape, np.uint8)
    ek, ev = oracle.reshape_and_cache_fp8(z, z, w.new_key, w.new_value, w.slot_mapping, bs, ks, vs)
    got_k, got_v = _codes(kc), _codes(vc)
    assert np.array_equal(got_k[s // bs, s % bs], ek[s // bs, s % bs])
    assert np.array_equal(got_v[s // bs, s % bs], ev[s // bs, s % bs])
    untouched = np.ones(shape[:2], bool)
    untouched[s // bs, s % bs] = False
    assert not got_k[untouched].any() and not got_v[untouched].any()


def test_fp8_write_empty_and_negative():
    w = workloads.make(1)
    kc = torch.full(w.key_cache.shape, 0x5A, dtype=U8, device="cuda")
    vc = kc.clone()
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    gp.reshape_and_cache_fp8(to_dev(w.new_key, BF), to_dev(w.new_value, BF), kc, vc, one, one,
                             torch.full((w.num_tokens,), -1, dtype=torch.int64, device="cuda"))
    empty = torch.empty((0, 1, 64), dtype=BF, device="cuda")
    gp.reshape_and_cache_fp8(empty, empty, kc, vc, one, one,
                             torch.empty((0,), dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert (_codes(kc) == 0x5A).all() and (_codes(vc) == 0x5A).all()


# ---------------------------------------------------------------------------
# Attention over E4M3 caches
# ---------------------------------------------------------------------------

class Fp8Case:
    """A workload's E4M3 caches: the GPU's (whole pool, written by the GPU) and the
    oracle's (quantised on the CPU: the blocks of ``seqs``, or the whole pool when
    ``seqs`` is None)."""

    def __init__(self, w, seqs=None):
        self.w, self.seqs = w, seqs
        self.ks, self.vs = _scales(w.key_cache), _scales(w.value_cache)
        d = Dev(w)
        self.d = d
        NB, bs, Hkv, D = w.key_cache.shape
        self.kc = torch.empty((NB, bs, Hkv, D), dtype=U8, device="cuda")
        self.vc = torch.empty_like(self.kc)
        self.d_ks = to_dev(self.ks, torch.float32)
        self.d_vs = to_dev(self.vs, torch.float32)
        all_slots = torch.arange(NB * bs, dtype=torch.int64, device="cuda")
        gp.reshape_and_cache_fp8(d.kc.view(NB * bs, Hkv, D), d.vc.view(NB * bs, Hkv, D), self.kc,
                                 self.vc, self.d_ks, self.d_vs, all_slots)
        torch.cuda.synchronize()
        if seqs is None:   # the whole pool, both sides
            self.okc = fp8_codes(w.key_cache, self.ks)
            self.ovc = fp8_codes(w.value_cache, self.vs)
            assert np.array_equal(self.kc.cpu().numpy(), self.okc), "GPU key codes differ"
            assert np.array_equal(self.vc.cpu().numpy(), self.ovc), "GPU value codes differ"
            return
        # the oracle's codes for the blocks the given sequences read
        self.okc = np.zeros((NB, bs, Hkv, D), np.uint8)
        self.ovc = np.zeros((NB, bs, Hkv, D), np.uint8)
        blocks = sorted({int(x) for b in seqs
                         for x in w.block_tables[b, :-(-int(w.context_lens[b]) // bs)]})
        blocks = np.array(blocks, dtype=np.int64)
        if blocks.size:
            self.okc[blocks] = oracle.quantize_fp8(w.key_cache[blocks], self.ks)
            self.ovc[blocks] = oracle.quantize_fp8(w.value_cache[blocks], self.vs)
            got_k = self.kc[torch.from_numpy(blocks).cuda()].cpu().numpy()
            got_v = self.vc[torch.from_numpy(blocks).cuda()].cpu().numpy()
            assert np.array_equal(got_k, self.okc[blocks]), "GPU key codes differ from the oracle"
            assert np.array_equal(got_v, self.ovc[blocks]), "GPU value codes differ from the oracle"

    def dense(self):
        w, d = self.w, self.d
        return gp.paged_attention_decode_fp8(d.q, self.kc, self.vc, self.d_ks, self.d_vs, d.bt,
                                             d.ctx, max_context_len=w.max_context_len,
                                             scale=float(w.scale)).cpu().numpy()

    def sparse(self, sel):
        w, d = self.w, self.d
        return gp.sparse_paged_attention_decode_fp8(
            d.q, self.kc, self.vc, self.d_ks, self.d_vs, d.bt, d.ctx, to_dev(sel, torch.int32),
            max_context_len=w.max_context_len, scale=float(w.scale)).cpu().numpy()

    def ref_dense(self):
        w = self.w
        return oracle.paged_attention_decode_fp8(w.query, self.okc, self.ovc, self.ks, self.vs,
                                                 w.block_tables, w.context_lens, w.scale,
                                                 seqs=self.seqs)


@functools.lru_cache(maxsize=None)
def _full_case(config):
    """Whole-pool E4M3 caches of a full-size workload (GPU and oracle), built once."""
    return Fp8Case(workload(config))


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_fp8_dense_config(config):
    w = workload(config)
    c = _full_case(config)
    out = c.dense()
    err = max_abs(out, c.ref_dense())
    print(f"config {config}: FP8 max-abs vs oracle {err:.3e} over all {w.batch} sequences")
    assert err <= ATOL


FP8_CASES = [
    (601, 4, 1, 64, 16, [0, 1, 15, 16, 17, 33]),
    (602, 28, 4, 128, 16, [31, 32, 33, 500, 1023, 1025]),
    (603, 16, 16, 128, 32, [7, 64, 65, 300]),
    (604, 16, 1, 128, 64, [129, 2047, 4100]),
    (605, 64, 8, 128, 128, [1, 127, 128, 129, 3000]),
    (606, 14, 2, 64, 128, [250, 1, 700]),
]


@pytest.mark.parametrize("schedule", ["balanced", "split"])
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx", FP8_CASES)
def test_fp8_dense_random(seed, Hq, Hkv, D, bs, ctx, schedule, monkeypatch):
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=ctx)
    c = Fp8Case(w, list(range(w.batch)))
    out = c.dense()
    err = max_abs(out, c.ref_dense())
    print(f"seed {seed}: FP8 max-abs {err:.3e}")
    assert err <= ATOL
    for b, L in enumerate(ctx):
        if L == 0:
            assert (out[b] == 0).all()


@functools.lru_cache(maxsize=None)
def _sparse_ref(config, K):
    w, c = workload(config), _full_case(config)
    return oracle.sparse_paged_attention_decode_fp8(w.query, c.okc, c.ovc, c.ks, c.vs,
                                                    w.block_tables, w.context_lens,
                                                    oracle_selection(config, K), w.scale)


@pytest.mark.parametrize("schedule", ["balanced", "split", "direct"])
@pytest.mark.parametrize("config,K", [(1, 3), (3, 64), (5, 32)])
def test_fp8_sparse_config(config, K, schedule, monkeypatch):
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workload(config)
    c = _full_case(config)
    out = c.sparse(oracle_selection(config, K))
    err = max_abs(out, _sparse_ref(config, K))
    print(f"config {config} K={K}: FP8 sparse max-abs {err:.3e} over all {w.batch} sequences")
    assert err <= ATOL


# ---------------------------------------------------------------------------
# The FP8 dense step in one call (decode append)
# ---------------------------------------------------------------------------

def _fp8_append_check(w, c):
    """paged_attention_decode_fp8_append on copies of the case's E4M3 caches against
    the oracle chain: the FP8 write of the new tokens, then FP8 dense attention."""
    assert w.num_tokens == w.batch, "decode append writes token b for sequence b"
    d = c.d
    kc, vc = c.kc.clone(), c.vc.clone()
    out = gp.paged_attention_decode_fp8_append(d.q, d.nk, d.nv, kc, vc, c.d_ks, c.d_vs, d.slots,
                                               d.bt, d.ctx, max_context_len=w.max_context_len,
                                               scale=float(w.scale))
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache_fp8(c.okc, c.ovc, w.new_key, w.new_value, w.slot_mapping,
                                          w.block_size, c.ks, c.vs)
    seqs = c.seqs
    if seqs is None:
        assert np.array_equal(kc.cpu().numpy(), ek), "key codes differ from the oracle"
        assert np.array_equal(vc.cpu().numpy(), ev), "value codes differ from the oracle"
    else:   # the oracle holds codes for the blocks the sequences read
        blocks = sorted({int(x) for b in seqs
                         for x in w.block_tables[b, :-(-int(w.context_lens[b]) // w.block_size)]})
        assert np.array_equal(kc.cpu().numpy()[blocks], ek[blocks]), "key codes differ"
        assert np.array_equal(vc.cpu().numpy()[blocks], ev[blocks]), "value codes differ"
    ref = oracle.paged_attention_decode_fp8(w.query, ek, ev, c.ks, c.vs, w.block_tables,
                                            w.context_lens, w.scale, seqs=seqs)
    err = max_abs(out.cpu().numpy(), ref)
    print(f"{w.name}: FP8 append max-abs vs oracle {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("schedule", ["balanced", "split"])
@pytest.mark.parametrize("config", [1, 2, 5])
def test_fp8_append_config(config, schedule, monkeypatch):
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    _fp8_append_check(workload(config), _full_case(config))


@pytest.mark.parametrize("schedule", ["balanced", "split"])
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx", [
    (631, 4, 1, 64, 16, [1, 2, 16, 17, 33]),
    (632, 28, 4, 128, 16, [31, 32, 5000, 1025]),
    (633, 64, 8, 128, 128, [1, 128, 129, 3000]),
])
def test_fp8_append_random(seed, Hq, Hkv, D, bs, ctx, schedule, monkeypatch):
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workloads.random_case(seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=bs, context_lens=ctx, num_tokens=len(ctx), neg_slots=1)
    _fp8_append_check(w, Fp8Case(w, list(range(w.batch))))


@pytest.mark.parametrize("schedule", ["balanced", "split"])
def test_fp8_append_spiked_new_token(schedule, monkeypatch):
    """The new key along each head's query (one query head per KV head), sized to carry
    about half of its sequence's softmax: its codes' scale and its unit's lse are
    checked at O(0.1) sensitivity."""
    from test_append_gpu import spike_keys
    monkeypatch.setenv("GPKV_ATTN_SCHEDULE", schedule)
    w = workloads.random_case(641, batch=3, num_q_heads=4, num_kv_heads=4, head_dim=128,
                              block_size=16, context_lens=[9000, 3000, 2], num_tokens=3)
    w.new_key[...] = spike_keys(w)
    _fp8_append_check(w, Fp8Case(w, list(range(w.batch))))
