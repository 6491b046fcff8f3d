"""GPU parity of multi-token queries (varlen, causal mask aligned to the right)
against the CPU oracle. Bar: max-abs 2e-3 (bf16 inputs, fp32 accumulation)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import BF, Dev, fp8_codes, max_abs, to_dev

pytestmark = pytest.mark.gpu
ATOL = 2e-3


def _run(w, **kw):
    d = Dev(w)
    qv = to_dev(w.query_varlen, BF)
    cu = to_dev(w.cu_seqlens_q, torch.int32)
    ql = np.diff(w.cu_seqlens_q)
    out = gp.paged_attention_varlen(qv, d.kc, d.vc, d.bt, d.ctx, cu, max_q_len=int(ql.max()),
                                    max_context_len=w.max_context_len, scale=float(w.scale), **kw)
    return d, out.cpu().numpy()


def _ref(w, seqs=None):
    return oracle.paged_attention_varlen(w.query_varlen, w.key_cache, w.value_cache,
                                         w.block_tables, w.context_lens, w.cu_seqlens_q, w.scale,
                                         seqs=seqs)


VARLEN_CASES = [
    # seed, Hq, Hkv, D, bs, ctx, q_lens
    (701, 28, 4, 128, 16, [900, 33, 2500, 16, 1200, 700], [1, 7, 64, 16, 3, 1]),
    (702, 4, 1, 64, 16, [0, 1, 15, 17, 40, 5], [3, 1, 15, 2, 40, 9]),      # q_len >= ctx rows
    (703, 16, 16, 128, 32, [300, 65, 1000], [2, 65, 200]),                   # G = 1
    (704, 16, 1, 128, 64, [129, 2047, 4100], [16, 1, 130]),                  # G = 16
    (705, 64, 8, 128, 128, [1, 127, 3000, 129], [1, 5, 100, 129]),
    (706, 14, 2, 64, 128, [250, 1, 700], [250, 1, 33]),
    (707, 12, 3, 64, 32, [513, 514, 96], [1, 2, 96]),
]


# Both schedules of the multi-token call: fixed KV splits, and equal shares of the
# flattened (unit, tile) space over the resident workgroups.
VARLEN_SCHEDULES = ["split", "balanced"]


@pytest.mark.parametrize("schedule", VARLEN_SCHEDULES)
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx,ql", VARLEN_CASES)
def test_varlen_random(seed, Hq, Hkv, D, bs, ctx, ql, schedule, monkeypatch):
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    w = workloads.varlen_case(seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                              context_lens=ctx, q_lens=ql)
    _, out = _run(w)
    ref = _ref(w)
    err = max_abs(out, ref)
    print(f"seed {seed}: varlen max-abs {err:.3e}")
    assert err <= ATOL
    assert (out[np.all(ref == 0, axis=(1, 2))] == 0).all(), "rows that see nothing are zero"


@pytest.mark.parametrize("split", [256, 2048, "balanced"])
def test_varlen_shared_tiles_at_the_causal_bound(split, monkeypatch):
    """Chunks on the shared-LDS path (at least four row tiles) whose first row's causal
    bound falls on a 32-position tile edge, one short of it and one past it, so that the
    last unmasked tile and the first masked one meet exactly there."""
    if split == "balanced":
        monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", "balanced")
    else:
        monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", "split")
        monkeypatch.setenv("GPKV_SPLIT_TOKENS", str(split))
    ctx = [1055, 1056, 1058, 2080, 96]
    ql = [32, 33, 31, 64, 96]          # first-row bounds 1024, 1024, 1028, 2017, 1
    w = workloads.varlen_case(721, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=ctx, q_lens=ql)
    _, out = _run(w)
    err = max_abs(out, _ref(w))
    print(f"split {split}: varlen max-abs {err:.3e}")
    assert err <= ATOL


def _shares_per_workgroup(B, total_q, Hq, Hkv, bs, max_ctx, cus):
    """The host's rule for the balanced schedule of the two-row-tile kernel: shares
    are a multiple of the grid (two workgroups per CU), each short enough that its
    blocks fit one staged table chunk of 2048 entries."""
    G = Hq // Hkv
    total_rt = (total_q * G + 15) // 16 + B
    u_bound = Hkv * ((total_rt + 7) // 8 + B) + (total_rt + 1) // 2 + B
    w_bound = u_bound * ((max_ctx + 31) // 32)
    seg_cap = (2048 - 1) * bs // 32 - 1
    need = (w_bound + seg_cap - 2) // (seg_cap - 1)
    grid = 2 * cus
    return max(1, -(-need // grid))


@pytest.mark.parametrize("schedule", VARLEN_SCHEDULES)
def test_varlen_several_shares_per_workgroup(schedule, monkeypatch):
    """A max_context_len far above the real contexts makes the host's bound on a share's
    table span ask for more shares than workgroups: each workgroup then takes a run of
    consecutive shares, most of them empty (the work is smaller than the shares), and
    the combine must skip the empty ones. Decode rows and shared-LDS chunks together."""
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    rng = np.random.default_rng(731)
    B = 64
    ctx = [int(x) for x in rng.integers(1, 900, size=B)]
    ql = [1] * B
    for i, q in ((3, 40), (17, 64), (40, 25)):   # >= 4 row tiles: the shared path
        ctx[i] = max(ctx[i], q + 200)
        ql[i] = q
    w = workloads.varlen_case(731, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=ctx, q_lens=ql)
    max_ctx = 40960
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per = _shares_per_workgroup(B, int(sum(ql)), 28, 4, 16, max_ctx, cus)
    print(f"shares per workgroup: {per}")
    if schedule == "balanced":
        assert per >= 2, "the shape no longer reaches several shares per workgroup"
    d = Dev(w)
    # a block table wide enough for max_context_len; entries past a sequence's blocks
    # are never read
    bt = np.full((B, max_ctx // 16), -1, dtype=np.int32)
    bt[:, : w.block_tables.shape[1]] = w.block_tables
    qv = to_dev(w.query_varlen, BF)
    cu = to_dev(w.cu_seqlens_q, torch.int32)
    out = gp.paged_attention_varlen(qv, d.kc, d.vc, to_dev(bt, torch.int32), d.ctx, cu,
                                    max_q_len=max(ql), max_context_len=max_ctx,
                                    scale=float(w.scale))
    err = max_abs(out.cpu().numpy(), _ref(w))
    print(f"{schedule}: varlen max-abs {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("split", [128, 256, 512, 2048])
def test_varlen_split_sizes(split, monkeypatch):
    """Chunks whose rows end in different splits of the KV range (split schedule)."""
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", "split")
    monkeypatch.setenv("GPKV_SPLIT_TOKENS", str(split))
    w = workloads.varlen_case(710, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=[4000, 2500, 129, 700], q_lens=[300, 1, 129, 20])
    _, out = _run(w)
    assert max_abs(out, _ref(w)) <= ATOL


@pytest.mark.parametrize("schedule", VARLEN_SCHEDULES)
def test_varlen_single_tokens_equal_decode(schedule, monkeypatch):
    """q_len = 1 everywhere: the same rows as the decode call."""
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    ctx = [900, 33, 2500, 16, 0, 700]
    w = workloads.varlen_case(711, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=ctx, q_lens=[1] * 6)
    d, out = _run(w)
    dec = gp.paged_attention_decode(to_dev(w.query_varlen, BF), d.kc, d.vc, d.bt, d.ctx,
                                    max_context_len=w.max_context_len,
                                    scale=float(w.scale)).cpu().numpy()
    ref = _ref(w)
    assert max_abs(out, ref) <= ATOL and max_abs(dec, ref) <= ATOL
    assert max_abs(out, dec) <= 1e-5


@pytest.mark.parametrize("schedule", VARLEN_SCHEDULES)
def test_varlen_mixed_batch_8k(schedule, monkeypatch):
    """An 8K-average batch in which a few sequences bring prefill chunks and the rest
    decode one token each; every query row against the oracle."""
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    rng = np.random.default_rng(712)
    ctx = np.clip(np.round(rng.normal(8192, 2048, 64)), 2048, 16384).astype(np.int32)
    ql = np.ones(64, np.int32)
    ql[:6] = [128, 256, 64, 512, 32, 128]
    w = workloads.varlen_case(712, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=ctx, q_lens=ql)
    _, out = _run(w)
    err = max_abs(out, _mixed_ref(w))
    print(f"mixed 8K batch ({schedule}): varlen max-abs {err:.3e} over all {out.shape[0]} query rows")
    assert err <= ATOL


_MIXED_REF = {}


def _mixed_ref(w):
    """The oracle over the mixed batch, computed once for both schedules."""
    if "ref" not in _MIXED_REF:
        _MIXED_REF["ref"] = _ref(w)
    return _MIXED_REF["ref"]


@pytest.mark.parametrize("schedule", VARLEN_SCHEDULES)
def test_varlen_bad_offsets_read_as_empty(schedule, monkeypatch):
    """A decreasing cu_seqlens entry makes that sequence empty; the others are
    unaffected and nothing outside the buffers is touched."""
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    w = workloads.varlen_case(713, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                              context_lens=[40, 50, 60], q_lens=[4, 3, 5])
    d = Dev(w)
    bad = np.array([0, 4, 2, 13], np.int32)   # sequence 1 decreasing; sequence 2 past total_q
    qv = to_dev(w.query_varlen, BF)
    out = torch.full((12, 8, 64), 7.0, device="cuda")
    gp.paged_attention_varlen(qv, d.kc, d.vc, d.bt, d.ctx, to_dev(bad, torch.int32), max_q_len=10,
                              max_context_len=w.max_context_len, scale=float(w.scale), out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = _ref(w)
    assert max_abs(got[:4], ref[:4]) <= ATOL          # sequence 0 intact
    assert (got[4:] == 7.0).all(), "rows of the empty sequences are not written"


# ---------------------------------------------------------------------------
# E4M3 caches: codes made on the CPU by the oracle's encoder, the same codes in
# both, attention compared (bar as above)
# ---------------------------------------------------------------------------

def _fp8_case(w):
    Hkv = w.num_kv_heads
    k = oracle.bf16_to_f64(w.key_cache)
    v = oracle.bf16_to_f64(w.value_cache)
    ks = (np.abs(k).max(axis=(0, 1, 3)) / 256.0).clip(min=1e-3).astype(np.float32)
    vs = (np.abs(v).max(axis=(0, 1, 3)) / 256.0).clip(min=1e-3).astype(np.float32)
    assert ks.shape == (Hkv,)
    kq = oracle.quantize_fp8(w.key_cache, ks)
    vq = oracle.quantize_fp8(w.value_cache, vs)
    return kq, vq, ks, vs


def _run_fp8(w, kq, vq, ks, vs):
    qv = to_dev(w.query_varlen, BF)
    ql = np.diff(w.cu_seqlens_q)
    out = gp.paged_attention_varlen_fp8(
        qv, to_dev(kq, torch.uint8), to_dev(vq, torch.uint8), to_dev(ks, torch.float32),
        to_dev(vs, torch.float32), to_dev(w.block_tables, torch.int32),
        to_dev(w.context_lens, torch.int32), to_dev(w.cu_seqlens_q, torch.int32),
        max_q_len=int(ql.max()), max_context_len=w.max_context_len, scale=float(w.scale))
    return out.cpu().numpy()


FP8_VARLEN_CASES = [
    # seed, Hq, Hkv, D, bs, ctx, q_lens
    (721, 28, 4, 128, 16, [900, 33, 2500, 16, 1200, 700], [1, 7, 64, 16, 3, 1]),
    (722, 4, 1, 64, 16, [0, 1, 15, 17, 40, 5], [3, 1, 15, 2, 40, 9]),
    (723, 16, 1, 128, 64, [129, 2047, 4100], [16, 1, 130]),
    (724, 14, 2, 64, 128, [250, 1, 700], [250, 1, 33]),
]


@pytest.mark.parametrize("schedule", VARLEN_SCHEDULES)
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs,ctx,ql", FP8_VARLEN_CASES)
def test_varlen_fp8_random(seed, Hq, Hkv, D, bs, ctx, ql, schedule, monkeypatch):
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    w = workloads.varlen_case(seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                              context_lens=ctx, q_lens=ql)
    kq, vq, ks, vs = _fp8_case(w)
    out = _run_fp8(w, kq, vq, ks, vs)
    ref = oracle.paged_attention_varlen_fp8(w.query_varlen, kq, vq, ks, vs, w.block_tables,
                                            w.context_lens, w.cu_seqlens_q, w.scale)
    err = max_abs(out, ref)
    print(f"seed {seed}: FP8 varlen max-abs {err:.3e}")
    assert err <= ATOL
    assert (out[np.all(ref == 0, axis=(1, 2))] == 0).all(), "rows that see nothing are zero"


def test_varlen_fp8_single_tokens_equal_fp8_decode():
    ctx = [900, 33, 2500, 16, 0, 700]
    w = workloads.varlen_case(725, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=ctx, q_lens=[1] * 6)
    kq, vq, ks, vs = _fp8_case(w)
    out = _run_fp8(w, kq, vq, ks, vs)
    dec = gp.paged_attention_decode_fp8(
        to_dev(w.query_varlen, BF), to_dev(kq, torch.uint8), to_dev(vq, torch.uint8),
        to_dev(ks, torch.float32), to_dev(vs, torch.float32), to_dev(w.block_tables, torch.int32),
        to_dev(w.context_lens, torch.int32), max_context_len=w.max_context_len,
        scale=float(w.scale)).cpu().numpy()
    assert max_abs(out, dec) <= 1e-5


@pytest.mark.parametrize("split", [256, 2048, "balanced"])
def test_varlen_fp8_shared_tiles_at_the_causal_bound(split, monkeypatch):
    """E4M3 chunks on the shared-LDS path (codes widened to bf16 as they are staged),
    with first-row causal bounds on, one short of and one past a 32-position tile edge."""
    if split == "balanced":
        monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", "balanced")
    else:
        monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", "split")
        monkeypatch.setenv("GPKV_SPLIT_TOKENS", str(split))
    w = workloads.varlen_case(726, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=[1055, 1056, 1058, 2080, 96],
                              q_lens=[32, 33, 31, 64, 96])
    kq, vq, ks, vs = _fp8_case(w)
    out = _run_fp8(w, kq, vq, ks, vs)
    ref = oracle.paged_attention_varlen_fp8(w.query_varlen, kq, vq, ks, vs, w.block_tables,
                                            w.context_lens, w.cu_seqlens_q, w.scale)
    err = max_abs(out, ref)
    print(f"split {split}: FP8 varlen max-abs {err:.3e}")
    assert err <= ATOL


_MIXED_FP8 = {}


@pytest.mark.parametrize("schedule", VARLEN_SCHEDULES)
def test_varlen_fp8_mixed_batch_8k(schedule, monkeypatch):
    """The 8K-average mixed batch over E4M3 caches (per-head scales amax / 256): the six
    chunks take the shared-LDS path, the single tokens the per-head one; every query row
    against the oracle on the same codes."""
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    if "case" not in _MIXED_FP8:
        rng = np.random.default_rng(714)
        ctx = np.clip(np.round(rng.normal(8192, 2048, 64)), 2048, 16384).astype(np.int32)
        ql = np.ones(64, np.int32)
        ql[:6] = [128, 256, 64, 512, 32, 128]
        w = workloads.varlen_case(714, num_q_heads=28, num_kv_heads=4, head_dim=128,
                                  block_size=16, context_lens=ctx, q_lens=ql)
        k = (w.key_cache.astype(np.uint32) << np.uint32(16)).view(np.float32)
        v = (w.value_cache.astype(np.uint32) << np.uint32(16)).view(np.float32)
        ks = np.maximum(np.abs(k).max(axis=(0, 1, 3)) / 256.0, 1e-3).astype(np.float32)
        vs = np.maximum(np.abs(v).max(axis=(0, 1, 3)) / 256.0, 1e-3).astype(np.float32)
        del k, v
        kq, vq = fp8_codes(w.key_cache, ks), fp8_codes(w.value_cache, vs)
        ref = oracle.paged_attention_varlen_fp8(w.query_varlen, kq, vq, ks, vs, w.block_tables,
                                                w.context_lens, w.cu_seqlens_q, w.scale)
        _MIXED_FP8["case"] = (w, kq, vq, ks, vs, ref)
    w, kq, vq, ks, vs, ref = _MIXED_FP8["case"]
    out = _run_fp8(w, kq, vq, ks, vs)
    err = max_abs(out, ref)
    print(f"mixed 8K batch, E4M3 ({schedule}): max-abs {err:.3e} over all {out.shape[0]} rows")
    assert err <= ATOL
