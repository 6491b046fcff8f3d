"""The whole decode step captured into a HIP graph: replay equals eager, bit for bit,
and both equal the oracle chain.

[TL18] 6.2 (TileLang tutorial ch. 18, graph capture): graph mode only removes the
host-side launch cost, so the check is that replays give exactly the eager results.
Every call launches on torch's current stream with a grid fixed by host scalars and
no memset, so it is capturable. Replays are interleaved with eager work and
synchronisations, and every replay is compared with the eager result; the eager
result itself (caches, metadata, Top-K ids, both attention outputs) is compared
with the CPU oracle's write -> metadata -> dense / select -> sparse chain (bits
exact, attention within 2e-3).
"""
import functools

import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import BF, Dev, bits, max_abs, to_dev

ATOL = 2e-3

pytestmark = pytest.mark.gpu


def _step_buffers(w, d, K):
    """Workspaces and outputs, and the prefill state: this step's tokens already in
    the cache and the metadata built over it, so that the step's write and its
    incremental metadata update are idempotent (every run leaves the same state)."""
    B, Hq, Hkv, D, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    mcl = w.max_context_len
    buf = {
        "out_d": torch.empty((B, Hq, D), dtype=torch.float32, device="cuda"),
        "out_s": torch.empty((B, Hq, D), dtype=torch.float32, device="cuda"),
        "ws_d": torch.zeros(gp.paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, mcl),
                            dtype=torch.uint8, device="cuda"),
        "ws_sel": torch.empty(gp.quest_select_workspace_bytes(B, Hkv, w.max_blocks_per_seq),
                              dtype=torch.uint8, device="cuda"),
        "ws_sp": torch.zeros(gp.sparse_attention_workspace_bytes(B, Hq, Hkv, D, bs, K),
                             dtype=torch.uint8, device="cuda"),
        "ws_qd": torch.zeros(gp.quest_decode_workspace_bytes(B, Hq, Hkv, D, bs,
                                                             w.max_blocks_per_seq, K),
                             dtype=torch.uint8, device="cuda"),
        "sel": torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda"),
        "kmin": torch.zeros((w.num_blocks, Hkv, D), dtype=BF, device="cuda"),
        "kmax": torch.zeros((w.num_blocks, Hkv, D), dtype=BF, device="cuda"),
    }
    gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, d.slots)
    gp.quest_block_metadata(d.kc, d.bt, d.ctx, buf["kmin"], buf["kmax"], max_context_len=mcl)
    return buf


def _graph_case(case):
    if case == "random":
        w = workloads.random_case(401, batch=6, num_q_heads=28, num_kv_heads=4, head_dim=128,
                                  block_size=16, context_lens=[900, 33, 2500, 16, 1200, 700],
                                  num_tokens=6, neg_slots=1)
        return w, 12
    if case == "long":   # few pairs, long selections
        w = workloads.random_case(403, batch=2, num_q_heads=28, num_kv_heads=4, head_dim=128,
                                  block_size=16, context_lens=[20000, 9000], num_tokens=2)
        return w, 200
    w = workloads.make(3)
    return w, w.topk_list[0]


@functools.lru_cache(maxsize=None)
def _oracle_chain(case):
    """The step on the CPU: write, metadata of the written cache, dense attention,
    Top-K, sparse attention over the selection."""
    w, K = _graph_case(case)
    bs = w.block_size
    kc, vc = oracle.reshape_and_cache(w.key_cache, w.value_cache, w.new_key, w.new_value,
                                      w.slot_mapping, bs)
    kmin, kmax = oracle.quest_block_metadata(kc, w.block_tables, w.context_lens, bs)
    sel = oracle.quest_select_topk(w.query, kmin, kmax, w.block_tables, w.context_lens, bs, K)
    return {"kc": kc, "vc": vc, "kmin": kmin, "kmax": kmax, "sel": sel,
            "out_d": oracle.paged_attention_decode(w.query, kc, vc, w.block_tables,
                                                   w.context_lens, w.scale),
            "out_s": oracle.sparse_paged_attention_decode(w.query, kc, vc, w.block_tables,
                                                          w.context_lens, sel, w.scale)}


def _meta_equal(got, exp, referenced):
    """Bitwise on the referenced blocks, +0 and -0 counted equal."""
    g, e = got[referenced].copy(), exp[referenced].copy()
    g[g == 0x8000] = 0
    e[e == 0x8000] = 0
    return np.array_equal(g, e)


def _check_against_oracle(case, w, snap):
    exp = _oracle_chain(case)
    assert np.array_equal(bits(snap["kc"]), exp["kc"]), "key cache differs from the oracle"
    assert np.array_equal(bits(snap["vc"]), exp["vc"]), "value cache differs from the oracle"
    referenced = np.unique(np.concatenate(
        [w.block_tables[b, :-(-int(L) // w.block_size)] for b, L in enumerate(w.context_lens)]))
    assert _meta_equal(bits(snap["kmin"]), exp["kmin"], referenced), "key_min differs"
    assert _meta_equal(bits(snap["kmax"]), exp["kmax"], referenced), "key_max differs"
    assert np.array_equal(snap["sel"].cpu().numpy(), exp["sel"]), "Top-K ids differ"
    err_d = max_abs(snap["out_d"].cpu().numpy(), exp["out_d"])
    err_s = max_abs(snap["out_s"].cpu().numpy(), exp["out_s"])
    print(f"{case}: dense max-abs {err_d:.3e}, sparse max-abs {err_s:.3e}")
    assert err_d <= ATOL and err_s <= ATOL


def _step(w, d, buf, K, fused, one_call=False):
    """fused: False (write, dense, metadata refresh), True (write with the metadata
    fold, dense) or "append" (write, fold and dense attention in one call)."""
    mcl, bs, scale = w.max_context_len, w.block_size, float(w.scale)
    if fused == "append":
        gp.paged_attention_decode_append(d.q, d.nk, d.nv, d.kc, d.vc, d.slots, d.bt, d.ctx,
                                         max_context_len=mcl, scale=scale, key_min=buf["kmin"],
                                         key_max=buf["kmax"], out=buf["out_d"],
                                         workspace=buf["ws_d"])
    else:
        if fused:   # write + incremental metadata in one launch (both idempotent)
            gp.reshape_and_cache_quest(d.nk, d.nv, d.kc, d.vc, buf["kmin"], buf["kmax"], d.slots)
        else:
            gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, d.slots)
        gp.paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx, max_context_len=mcl, scale=scale,
                                  out=buf["out_d"], workspace=buf["ws_d"])
    if not fused:
        gp.quest_block_metadata(d.kc, d.bt, d.ctx, buf["kmin"], buf["kmax"],
                                max_context_len=mcl, last_block_only=True)
    if one_call:
        gp.quest_decode(d.q, d.kc, d.vc, buf["kmin"], buf["kmax"], d.bt, d.ctx, topk_blocks=K,
                        max_context_len=mcl, scale=scale, out=buf["out_s"], topk_out=buf["sel"],
                        workspace=buf["ws_qd"])
        return
    gp.quest_select_topk(d.q, buf["kmin"], buf["kmax"], d.bt, d.ctx, block_size=bs,
                         topk_blocks=K, max_context_len=mcl, out=buf["sel"],
                         workspace=buf["ws_sel"])
    gp.sparse_paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx, buf["sel"],
                                     max_context_len=mcl, scale=scale, out=buf["out_s"],
                                     workspace=buf["ws_sp"])


def _snapshot(buf, d):
    return {k: v.clone() for k, v in (("out_d", buf["out_d"]), ("out_s", buf["out_s"]),
                                      ("sel", buf["sel"]), ("kmin", buf["kmin"]),
                                      ("kmax", buf["kmax"]), ("kc", d.kc), ("vc", d.vc))}


@pytest.mark.parametrize("case,fused,one_call", [("random", False, False), ("config3", False, False),
                                                 ("random", True, False), ("config3", True, False),
                                                 ("random", True, "fused"), ("config3", True, "fused"),
                                                 ("long", True, "auto"),
                                                 ("long", True, "fused"),
                                                 ("random", "append", False),
                                                 ("config3", "append", "fused"),
                                                 ("long", "append", "auto")])
def test_graph_replay_equals_eager(case, fused, one_call, monkeypatch):
    if one_call:   # the one-call Quest decode on the path named
        monkeypatch.setenv("GPKV_QUEST_DECODE_PATH", one_call)
    w, K = _graph_case(case)
    d = Dev(w)
    buf = _step_buffers(w, d, K)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on the capture stream
        _step(w, d, buf, K, fused, one_call)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _step(w, d, buf, K, fused, one_call)       # eager reference (the write is idempotent)
    torch.cuda.synchronize()
    ref = _snapshot(buf, d)
    _check_against_oracle(case, w, ref)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, d, buf, K, fused, one_call)
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(4):
        # eager work between replays: clobber the outputs, then replay
        buf["out_d"].fill_(float("nan"))
        buf["out_s"].fill_(float("nan"))
        buf["sel"].fill_(-7)
        scratch.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(buf, d)
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs from eager"


@pytest.mark.parametrize("schedule", ["split", "balanced"])
def test_graph_replay_varlen_equals_eager(schedule, monkeypatch):
    """The multi-token call (chunks on the LDS-shared path, single tokens on the
    per-head path, and its combine) captured and replayed: equal to eager."""
    monkeypatch.setenv("GPKV_VARLEN_SCHEDULE", schedule)
    w = workloads.varlen_case(402, num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                              context_lens=[900, 33, 2500, 16, 1200, 700],
                              q_lens=[1, 7, 64, 16, 3, 1])
    d = Dev(w)
    qv = to_dev(w.query_varlen, BF)
    cu = to_dev(w.cu_seqlens_q, torch.int32)
    mq = int(np.diff(w.cu_seqlens_q).max())
    out = torch.empty((qv.shape[0], w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    ws = torch.empty(gp.paged_attention_varlen_workspace_bytes(
        w.batch, qv.shape[0], mq, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
        w.max_context_len), dtype=torch.uint8, device="cuda")

    def call():
        gp.paged_attention_varlen(qv, d.kc, d.vc, d.bt, d.ctx, cu, max_q_len=mq,
                                  max_context_len=w.max_context_len, scale=float(w.scale),
                                  out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xAB)                  # stale partial rows must not leak into a replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from eager"


# ---------------------------------------------------------------------------
# The step over E4M3 caches (Quest with code metadata)
# ---------------------------------------------------------------------------

def _fp8_step(w, c, buf, K, one_call):
    """The FP8 step: one_call -- quest_decode_fp8_append (write, code fold, selection,
    sparse attention) then the FP8 dense call; else the write with the code fold, the
    FP8 dense call, the FP8 selection and FP8 sparse attention."""
    d, mcl, bs, scale = c.d, w.max_context_len, w.block_size, float(w.scale)
    if one_call:
        gp.quest_decode_fp8_append(d.q, d.nk, d.nv, c.kc, c.vc, c.d_ks, c.d_vs, buf["kmin"],
                                   buf["kmax"], d.slots, d.bt, d.ctx, topk_blocks=K,
                                   max_context_len=mcl, scale=scale, out=buf["out_s"],
                                   topk_out=buf["sel"], workspace=buf["ws_qd"])
        gp.paged_attention_decode_fp8(d.q, c.kc, c.vc, c.d_ks, c.d_vs, d.bt, d.ctx,
                                      max_context_len=mcl, scale=scale, out=buf["out_d"],
                                      workspace=buf["ws_d"])
        return
    gp.reshape_and_cache_fp8_quest(d.nk, d.nv, c.kc, c.vc, c.d_ks, c.d_vs, buf["kmin"],
                                   buf["kmax"], d.slots)
    gp.paged_attention_decode_fp8(d.q, c.kc, c.vc, c.d_ks, c.d_vs, d.bt, d.ctx,
                                  max_context_len=mcl, scale=scale, out=buf["out_d"],
                                  workspace=buf["ws_d"])
    gp.quest_select_topk_fp8(d.q, buf["kmin"], buf["kmax"], d.bt, d.ctx, block_size=bs,
                             topk_blocks=K, max_context_len=mcl, out=buf["sel"],
                             workspace=buf["ws_sel"])
    gp.sparse_paged_attention_decode_fp8(d.q, c.kc, c.vc, c.d_ks, c.d_vs, d.bt, d.ctx,
                                         buf["sel"], max_context_len=mcl, scale=scale,
                                         out=buf["out_s"], workspace=buf["ws_sp"])


@pytest.mark.parametrize("case,one_call", [("random", False), ("random", True), ("long", True)])
def test_graph_replay_fp8_equals_eager(case, one_call):
    """The FP8 step captured and replayed four times between eager work: every output,
    cache and code-metadata buffer equals eager bit for bit, and eager equals the
    oracle's FP8 chain (write, code metadata, Top-K, dense and sparse attention)."""
    from test_fp8_gpu import Fp8Case
    w, K = _graph_case(case)
    c = Fp8Case(w, list(range(w.batch)))
    d = c.d
    buf = _step_buffers_fp8(w, c, K)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _fp8_step(w, c, buf, K, one_call)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _fp8_step(w, c, buf, K, one_call)
    torch.cuda.synchronize()
    snap = lambda: {k: v.clone() for k, v in (("out_d", buf["out_d"]), ("out_s", buf["out_s"]),
                                               ("sel", buf["sel"]), ("kmin", buf["kmin"]),
                                               ("kmax", buf["kmax"]), ("kc", c.kc), ("vc", c.vc))}
    ref = snap()

    bs = w.block_size
    ek, ev = oracle.reshape_and_cache_fp8(c.okc, c.ovc, w.new_key, w.new_value, w.slot_mapping,
                                          bs, c.ks, c.vs)
    omin, omax = oracle.quest_block_metadata_fp8(ek, w.block_tables, w.context_lens, bs)
    osel = oracle.quest_select_topk_fp8(w.query, omin, omax, w.block_tables, w.context_lens, bs, K)
    referenced = np.unique(np.concatenate(
        [w.block_tables[b, :-(-int(L) // bs)] for b, L in enumerate(w.context_lens)]))
    for name, exp in (("kc", ek), ("vc", ev)):
        assert np.array_equal(ref[name].cpu().numpy()[referenced], exp[referenced]), name
    for name, exp in (("kmin", omin), ("kmax", omax)):
        g, e = ref[name].cpu().numpy()[referenced], exp[referenced].copy()
        g[g == 0x80] = 0
        e[e == 0x80] = 0
        assert np.array_equal(g, e), name
    assert np.array_equal(ref["sel"].cpu().numpy(), osel), "Top-K ids differ"
    err_d = max_abs(ref["out_d"].cpu().numpy(),
                    oracle.paged_attention_decode_fp8(w.query, ek, ev, c.ks, c.vs, w.block_tables,
                                                      w.context_lens, w.scale))
    err_s = max_abs(ref["out_s"].cpu().numpy(),
                    oracle.sparse_paged_attention_decode_fp8(w.query, ek, ev, c.ks, c.vs,
                                                             w.block_tables, w.context_lens, osel,
                                                             w.scale))
    print(f"{case} FP8: dense max-abs {err_d:.3e}, sparse max-abs {err_s:.3e}")
    assert err_d <= ATOL and err_s <= ATOL

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _fp8_step(w, c, buf, K, one_call)
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(4):
        buf["out_d"].fill_(float("nan"))
        buf["out_s"].fill_(float("nan"))
        buf["sel"].fill_(-7)
        scratch.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs from eager"


def _step_buffers_fp8(w, c, K):
    """The FP8 step's buffers and its prefill state: this step's tokens already in the
    E4M3 caches and the code metadata built over them (the step is then idempotent)."""
    B, Hq, Hkv, D, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    d, mcl = c.d, w.max_context_len
    buf = {
        "out_d": torch.empty((B, Hq, D), dtype=torch.float32, device="cuda"),
        "out_s": torch.empty((B, Hq, D), dtype=torch.float32, device="cuda"),
        "ws_d": torch.zeros(gp.paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, mcl),
                            dtype=torch.uint8, device="cuda"),
        "ws_sel": torch.empty(gp.quest_select_workspace_bytes(B, Hkv, w.max_blocks_per_seq),
                              dtype=torch.uint8, device="cuda"),
        "ws_sp": torch.zeros(gp.sparse_attention_workspace_bytes(B, Hq, Hkv, D, bs, K),
                             dtype=torch.uint8, device="cuda"),
        "ws_qd": torch.zeros(gp.quest_decode_workspace_bytes(B, Hq, Hkv, D, bs,
                                                             w.max_blocks_per_seq, K),
                             dtype=torch.uint8, device="cuda"),
        "sel": torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda"),
        "kmin": torch.zeros((w.num_blocks, Hkv, D), dtype=torch.uint8, device="cuda"),
        "kmax": torch.zeros((w.num_blocks, Hkv, D), dtype=torch.uint8, device="cuda"),
    }
    gp.reshape_and_cache_fp8(d.nk, d.nv, c.kc, c.vc, c.d_ks, c.d_vs, d.slots)
    gp.quest_block_metadata_fp8(c.kc, d.bt, d.ctx, buf["kmin"], buf["kmax"], max_context_len=mcl)
    return buf
