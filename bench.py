"""Decode-step benchmark of the paged GQA attention library on one MI355X.

One step = the whole hot path once over one batch of synthetic input:
  paged_attention_decode_append (dense attention, split-KV + combine, with the
  step's write: one new token per sequence, stored by the combine, which also folds
  it into its block's Quest min / max)
  -> quest_decode (Quest block selection and sparse attention over the selection;
  one launch when the batch's (sequence, KV head) pairs fill the GPU).
With --write-path fused the write is a launch of its own first
(reshape_and_cache_quest) and the dense call is paged_attention_decode; a workload
whose new tokens are not one per sequence takes that form, and one without new
tokens has no write. With --quest-path separate the Quest call is quest_select_topk
followed by sparse_paged_attention_decode (the two calls are also timed on their
own either way). With --write-path separate the first call is reshape_and_cache, a
quest_block_metadata refresh of each sequence's last block follows the dense call,
and the Quest part runs as the two separate calls.
Inputs are resident in HBM before timing. Before every timed step a 1 GiB buffer
is written so that no KV bytes survive in the 256 MB Infinity Cache; the
per-call durations come from HIP events on the launch stream and exclude that
flush. The value reported is the step's algorithmic KV/metadata bytes divided by
the step time (GB/s). The full metadata rebuild is a prefill-time cost and is
reported separately, outside the step. The one-call Quest decode is also timed
alone behind its own flush, and the Quest step is that call with the write folded
into it (quest_decode_append) timed alone, or the write plus quest_decode alone.

After the headline workload, a per-workload block times every call of each of the
five workloads alone behind the flush (write, dense call, one-call Quest decode),
with the dense and Quest step times and their fraction of peak HBM bandwidth.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_CONFIG = 3
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = "attn_balanced_dense_long8k_traffic.md"
def dominant_kernel(num_kv_heads: int) -> str:
    """The dense split kernel's instance: eight waves per workgroup with 8 KV heads or a
    multiple, four otherwise."""
    return f"attn_balanced_kernel<128, false, false, {8 if num_kv_heads % 8 == 0 else 4}>"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for PMC byte calibration)")
    ap.add_argument("--write-path", choices=["append", "fused", "separate"], default="append",
                    help="append: the write (and metadata fold) inside the dense call, "
                         "paged_attention_decode_append; fused: reshape_and_cache_quest; "
                         "separate: reshape_and_cache + quest_block_metadata(last_block_only)")
    ap.add_argument("--quest-path", choices=["one_call", "separate"], default="one_call",
                    help="Quest part of the step: quest_decode, or select + sparse calls")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 (E4M3) cache timing")
    ap.add_argument("--no-varlen", action="store_true", help="skip the multi-token query timing")
    ap.add_argument("--details", action="store_true", help="print per-call timings to stderr")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-workload block (configs 1-5, each call timed alone)")
    return ap.parse_args()


def strip_c_comments(text: str) -> str:
    """C / C++ source without comments, whitespace runs collapsed to one space (string
    and character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_hash(read=None) -> str:
    """Hash of the attention kernels' code (comments and layout ignored): the
    committed counters stay valid across comment-only edits and no longer."""
    h = hashlib.sha256()
    for f in ("paged_attention.hip", "attention.h", "gpkv_internal.h"):
        if read is None:
            with open(os.path.join(ROOT, "gqa_paged_kv_amd", "csrc", f), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(strip_c_comments(text).encode())
    return h.hexdigest()[:16]


def committed_traffic(cfg: int):
    """HBM bytes per launch of the dominant kernel from the committed PMC summary,
    or None when the summary is missing, for another workload, or the kernel source
    changed since the counters were taken."""
    path = os.path.join(PROFILES, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_cfg = re.search(r"workload_config:\s*(\d+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_cfg and m_bytes):
        return None
    if m_hash.group(1) != kernel_source_hash() or int(m_cfg.group(1)) != cfg:
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, target_s: float):
    """Time the CPU oracle on the first sequences of the same workload until about
    target_s seconds of work; report algorithmic GB/s of that sample."""
    import numpy as np
    import oracle
    from gqa_paged_kv_amd import roofline as R

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    K = w.topk_list[0] if w.topk_list else None
    kc, vc = w.key_cache, w.value_cache
    kmin = kmax = None
    if K:   # prefill-time metadata of every block (outside the step, as on the GPU)
        kmin, kmax = oracle.quest_block_metadata(kc, w.block_tables, w.context_lens, w.block_size)
    t0 = time.perf_counter()
    total_bytes = 0
    seqs_done = 0
    passes = 0
    # Whole passes over the workload (a pass is the full step), the last one cut
    # short once about target_s seconds of CPU work are done.
    while True:
        passes += 1
        kc, vc = w.key_cache, w.value_cache
        if w.num_tokens:
            kc, vc = oracle.reshape_and_cache(kc, vc, w.new_key, w.new_value, w.slot_mapping,
                                              w.block_size)
            total_bytes += R.write_bytes(w.slot_mapping, w.num_blocks, w.block_size,
                                         w.num_kv_heads, w.head_dim)
        for b in range(w.batch):
            ctx1 = w.context_lens[b:b + 1]
            bt1 = w.block_tables[b:b + 1]
            oracle.paged_attention_decode(w.query[b:b + 1], kc, vc, bt1, ctx1, w.scale)
            total_bytes += R.dense_attention_bytes(ctx1, w.num_kv_heads, w.head_dim)
            if K:
                kmin, kmax = oracle.quest_block_metadata(kc, bt1, ctx1, w.block_size,
                                                         last_block_only=True, key_min=kmin,
                                                         key_max=kmax)
                sel = oracle.quest_select_topk(w.query[b:b + 1], kmin, kmax, bt1, ctx1,
                                               w.block_size, K)
                oracle.sparse_paged_attention_decode(w.query[b:b + 1], kc, vc, bt1, ctx1, sel,
                                                     w.scale)
                total_bytes += (R.metadata_step_bytes(ctx1, w.block_size, w.num_kv_heads, w.head_dim)
                                + R.select_bytes(ctx1, w.block_size, w.num_kv_heads, w.head_dim)
                                + R.sparse_attention_bytes(sel, ctx1, w.block_size, w.head_dim))
            seqs_done += 1
            if time.perf_counter() - t0 >= target_s:
                break
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(total_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full decode steps (write + dense + Quest) of the same workload, float64 "
                      f"numpy: {seqs_done} sequence-steps ({passes} pass(es) over {w.batch} "
                      f"sequences), {dt:.1f} s"}


def time_alone(fn, flush, stream, steps):
    """Mean / median / min of one call timed with HIP events on the launch stream,
    each run behind a write of the flush buffer (after three untimed calls)."""
    import numpy as np
    import torch
    for _ in range(3):
        fn()
    ts = []
    for k in range(steps):
        flush.fill_(k & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    t = np.array(ts)
    return {"us_mean": round(float(t.mean()), 2), "us_median": round(float(np.median(t)), 2),
            "us_min": round(float(t.min()), 2)}


def per_config_block(cfg, flush, stream, steps):
    """Every call of one workload's decode step, each timed alone behind the flush:
    the write (when the workload has new tokens), the dense call and the one-call
    Quest decode (when it sets topk_blocks). Step figures are sums of those calls."""
    import numpy as np
    import torch

    import gqa_paged_kv_amd as gp
    import workloads
    from gqa_paged_kv_amd import roofline as R

    w = workloads.make(cfg)
    bf = torch.bfloat16

    def dev(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == bf:
            return torch.from_numpy(a.view(np.int16)).view(bf).cuda()
        return torch.from_numpy(a).to(dtype).cuda()
    kc, vc = dev(w.key_cache, bf), dev(w.value_cache, bf)
    q = dev(w.query, bf)
    bt, ctx = dev(w.block_tables, torch.int32), dev(w.context_lens, torch.int32)
    B, Hq, Hkv, D, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    mcl, scale = w.max_context_len, float(w.scale)
    K = w.topk_list[0] if w.topk_list else 0
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(gp.paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, mcl), dtype=torch.uint8,
                     device="cuda")
    res = {"workload": w.name, "sum_context": int(w.context_lens.sum()), "topk_blocks": K or None}
    write_us = 0.0
    kmin = kmax = None
    if w.num_tokens:
        nk, nv = dev(w.new_key, bf), dev(w.new_value, bf)
        slots = dev(w.slot_mapping, torch.int64)
        if K:
            kmin = torch.zeros((w.num_blocks, Hkv, D), dtype=bf, device="cuda")
            kmax = torch.zeros_like(kmin)
            gp.reshape_and_cache(nk, nv, kc, vc, slots)   # the step's tokens, then metadata:
            gp.quest_block_metadata(kc, bt, ctx, kmin, kmax, max_context_len=mcl)   # idempotent
            t = time_alone(lambda: gp.reshape_and_cache_quest(nk, nv, kc, vc, kmin, kmax, slots),
                           flush, stream, steps)
            res["write_call"] = "reshape_and_cache_quest"
        else:
            t = time_alone(lambda: gp.reshape_and_cache(nk, nv, kc, vc, slots), flush, stream,
                           steps)
            res["write_call"] = "reshape_and_cache"
        res["write_us"] = t["us_mean"]
        write_us = t["us_mean"]
    t = time_alone(lambda: gp.paged_attention_decode(q, kc, vc, bt, ctx, max_context_len=mcl,
                                                     scale=scale, out=out, workspace=ws),
                   flush, stream, steps)
    db = R.dense_attention_bytes(w.context_lens, Hkv, D)
    res["dense_call_us"] = t["us_mean"]
    res["dense_bytes"] = int(db)
    res["dense_gbps"] = round(db / (t["us_mean"] * 1e-6) / 1e9, 1)
    res["dense_pct_of_peak"] = round(100 * res["dense_gbps"] / R.MI355X_HBM_GBPS, 1)
    res["dense_step_us"] = round(write_us + t["us_mean"], 2)
    if w.num_tokens and w.num_tokens == B:   # the same dense step as one call (decode append)
        t = time_alone(lambda: gp.paged_attention_decode_append(
            q, nk, nv, kc, vc, slots, bt, ctx, max_context_len=mcl, scale=scale, key_min=kmin,
            key_max=kmax, out=out, workspace=ws), flush, stream, steps)
        res["dense_step_append_us"] = t["us_mean"]
    if K:
        if kmin is None:
            kmin = torch.zeros((w.num_blocks, Hkv, D), dtype=bf, device="cuda")
            kmax = torch.zeros_like(kmin)
            gp.quest_block_metadata(kc, bt, ctx, kmin, kmax, max_context_len=mcl)
        sel = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
        out_s = torch.empty_like(out)
        wq = torch.empty(gp.quest_decode_workspace_bytes(B, Hq, Hkv, D, bs, w.max_blocks_per_seq, K),
                         dtype=torch.uint8, device="cuda")
        t = time_alone(lambda: gp.quest_decode(q, kc, vc, kmin, kmax, bt, ctx, topk_blocks=K,
                                               max_context_len=mcl, scale=scale, out=out_s,
                                               topk_out=sel, workspace=wq),
                       flush, stream, steps)
        qb = (R.select_bytes(w.context_lens, bs, Hkv, D)
              + R.sparse_attention_bytes(sel.cpu().numpy(), w.context_lens, bs, D))
        if w.num_tokens and w.num_tokens == B:   # the Quest step as one call (decode append)
            ta = time_alone(lambda: gp.quest_decode_append(
                q, nk, nv, kc, vc, kmin, kmax, slots, bt, ctx, topk_blocks=K, max_context_len=mcl,
                scale=scale, out=out_s, topk_out=sel, workspace=wq), flush, stream, steps)
            res["quest_step_append_us"] = ta["us_mean"]
        res["quest_call_us"] = t["us_mean"]
        res["quest_bytes"] = int(qb)
        res["quest_gbps"] = round(qb / (t["us_mean"] * 1e-6) / 1e9, 1)
        res["quest_pct_of_peak"] = round(100 * res["quest_gbps"] / R.MI355X_HBM_GBPS, 1)
        res["quest_step_us"] = round(write_us + t["us_mean"], 2)
        res["quest_step_speedup_vs_dense_step"] = round(res["dense_step_us"] / res["quest_step_us"], 2)
        # The same Quest call over E4M3 copies of the caches and their code metadata.
        kc8, vc8, ks8, vs8 = fp8_copy(gp, kc, vc)
        kmin8 = torch.empty(kmin.shape, dtype=torch.uint8, device="cuda")
        kmax8 = torch.empty_like(kmin8)
        gp.quest_block_metadata_fp8(kc8, bt, ctx, kmin8, kmax8, max_context_len=mcl)
        t = time_alone(lambda: gp.quest_decode_fp8(q, kc8, vc8, ks8, vs8, kmin8, kmax8, bt, ctx,
                                                   topk_blocks=K, max_context_len=mcl,
                                                   scale=scale, out=out_s, topk_out=sel,
                                                   workspace=wq), flush, stream, steps)
        qb8 = (R.select_bytes(w.context_lens, bs, Hkv, D, elem_bytes=1)
               + R.sparse_attention_bytes(sel.cpu().numpy(), w.context_lens, bs, D, elem_bytes=1))
        res["quest_fp8_call_us"] = t["us_mean"]
        res["quest_fp8_gbps"] = round(qb8 / (t["us_mean"] * 1e-6) / 1e9, 1)
        del kc8, vc8, kmin8, kmax8
    del kc, vc, q, bt, ctx, out, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def fp8_copy(gp, kc, vc):
    """E4M3 copies of bf16 caches written by the FP8 write call over every slot, with
    per-KV-head scales amax / 256 (the largest values land near 256 of E4M3's 448)."""
    import torch
    NB, bs, Hkv, D = kc.shape

    def amax_scale(t):
        return (t.float().abs().amax(dim=(0, 1, 3)) / 256.0).clamp_min(1e-3).contiguous()
    ks8, vs8 = amax_scale(kc), amax_scale(vc)
    kc8 = torch.empty(kc.shape, dtype=torch.uint8, device="cuda")
    vc8 = torch.empty_like(kc8)
    gp.reshape_and_cache_fp8(kc.view(NB * bs, Hkv, D), vc.view(NB * bs, Hkv, D), kc8, vc8, ks8,
                             vs8, torch.arange(NB * bs, dtype=torch.int64, device="cuda"))
    return kc8, vc8, ks8, vs8


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs on one GPU and has no multi-GPU path (got --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gqa_paged_kv_amd as gp
    import workloads
    from gqa_paged_kv_amd import roofline as R

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w = workloads.make(args.config)
    print(f"[bench] workload {w.name}: {workloads.shape_summary(w)}", file=sys.stderr, flush=True)

    def dev(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == torch.bfloat16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).to(dtype).cuda()

    bf = torch.bfloat16
    kc, vc = dev(w.key_cache, bf), dev(w.value_cache, bf)
    q = dev(w.query, bf)
    bt, ctx = dev(w.block_tables, torch.int32), dev(w.context_lens, torch.int32)
    nk, nv = dev(w.new_key, bf), dev(w.new_value, bf)
    slots = dev(w.slot_mapping, torch.int64)
    B, Hq, Hkv, D, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    mcl = w.max_context_len
    K = w.topk_list[0] if w.topk_list else 0
    scale = float(w.scale)

    out_d = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    out_s = torch.empty_like(out_d)
    ws_d = torch.zeros(gp.paged_attention_workspace_bytes(B, Hq, Hkv, D, bs, mcl), dtype=torch.uint8,
                       device="cuda")
    kmin = torch.zeros((w.num_blocks, Hkv, D), dtype=bf, device="cuda")
    kmax = torch.zeros_like(kmin)
    if K:
        ws_sel = torch.empty(gp.quest_select_workspace_bytes(B, Hkv, w.max_blocks_per_seq),
                             dtype=torch.uint8, device="cuda")
        ws_sp = torch.zeros(gp.sparse_attention_workspace_bytes(B, Hq, Hkv, D, bs, K),
                            dtype=torch.uint8, device="cuda")
        sel = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
        ws_qd = torch.zeros(gp.quest_decode_workspace_bytes(B, Hq, Hkv, D, bs, w.max_blocks_per_seq,
                                                            K), dtype=torch.uint8, device="cuda")
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    # The one-call dense step needs one new token per sequence (token b is sequence b's
    # newest); other workloads take the separate write kernel.
    write_mode = args.write_path
    if write_mode == "append" and not (w.num_tokens and w.num_tokens == B):
        write_mode = "fused"
    fused = bool(K) and write_mode in ("fused", "append")
    one_call = fused and args.quest_path == "one_call"
    dense_name = "paged_attention_decode_append" if write_mode == "append" else "paged_attention_decode"
    if write_mode == "append":
        calls = [dense_name] + (["quest_decode"] if one_call else
                                (["quest_select_topk", "sparse_paged_attention_decode"] if K else []))
    elif one_call:
        calls = ["reshape_and_cache_quest", "paged_attention_decode", "quest_decode"]
    elif fused:
        calls = ["reshape_and_cache_quest", "paged_attention_decode", "quest_select_topk",
                 "sparse_paged_attention_decode"]
    elif K:
        calls = ["reshape_and_cache", "paged_attention_decode", "quest_block_metadata",
                 "quest_select_topk", "sparse_paged_attention_decode"]
    else:
        calls = ["reshape_and_cache", "paged_attention_decode"]
    if not w.num_tokens:   # a workload without new tokens has no write in its step
        calls = [c for c in calls if not c.startswith("reshape_and_cache")]

    def run_call(name):
        if name == "reshape_and_cache":
            if w.num_tokens:
                gp.reshape_and_cache(nk, nv, kc, vc, slots)
        elif name == "reshape_and_cache_quest":
            if w.num_tokens:
                gp.reshape_and_cache_quest(nk, nv, kc, vc, kmin, kmax, slots)
        elif name == "paged_attention_decode":
            gp.paged_attention_decode(q, kc, vc, bt, ctx, max_context_len=mcl, scale=scale,
                                      out=out_d, workspace=ws_d)
        elif name == "paged_attention_decode_append":
            gp.paged_attention_decode_append(q, nk, nv, kc, vc, slots, bt, ctx,
                                             max_context_len=mcl, scale=scale,
                                             key_min=kmin if K else None,
                                             key_max=kmax if K else None, out=out_d,
                                             workspace=ws_d)
        elif name == "quest_block_metadata":
            gp.quest_block_metadata(kc, bt, ctx, kmin, kmax, max_context_len=mcl, last_block_only=True)
        elif name == "quest_select_topk":
            gp.quest_select_topk(q, kmin, kmax, bt, ctx, block_size=bs, topk_blocks=K,
                                 max_context_len=mcl, out=sel, workspace=ws_sel)
        elif name == "sparse_paged_attention_decode":
            gp.sparse_paged_attention_decode(q, kc, vc, bt, ctx, sel, max_context_len=mcl,
                                             scale=scale, out=out_s, workspace=ws_sp)
        elif name == "quest_decode":
            gp.quest_decode(q, kc, vc, kmin, kmax, bt, ctx, topk_blocks=K, max_context_len=mcl,
                            scale=scale, out=out_s, topk_out=sel, workspace=ws_qd)

    def step(events=None):
        for i, name in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            run_call(name)
        if events is not None:
            events[len(calls)].record(stream)

    # Prefill-time work: full metadata build (timed once, outside the step), over a
    # cache that already holds this step's tokens, so that the step's incremental
    # update (idempotent) leaves exactly the metadata of the written cache.
    t_full = None
    if K:
        if w.num_tokens:
            gp.reshape_and_cache(nk, nv, kc, vc, slots)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flush.fill_(1)
        e0.record(stream)
        gp.quest_block_metadata(kc, bt, ctx, kmin, kmax, max_context_len=mcl, last_block_only=False)
        e1.record(stream)
        torch.cuda.synchronize()
        t_full = e0.elapsed_time(e1) * 1e3

    # Warm-up: at least `warmup` steps and at least 25 ms of work.
    torch.cuda.synchronize()
    tw = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or (time.perf_counter() - tw) < 0.025:
        step()
        n_warm += 1
        if n_warm % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(f"[bench] warm-up done: {n_warm} steps", file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(3)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        flush.fill_(k & 0xFF)
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    # The same step captured into one HIP graph (TileLang tutorial ch. 18, section
    # 6.2: replay removes the host launch cost only); timed separately, flushed alike.
    graph_us = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gts = []
        for k in range(args.steps):
            flush.fill_(k & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            gts.append(e0.elapsed_time(e1) * 1e3)
        graph_us = float(np.mean(gts))
        del g
    except RuntimeError as exc:   # report, do not fail the eager measurement
        print(f"[bench] graph capture unavailable: {exc}", file=sys.stderr)

    # The one-call Quest part timed alone behind its own flush, and as its two separate
    # calls, each alone (same flush).
    quest_separate = None
    quest_alone = None
    if one_call:
        quest_alone = time_alone(lambda: run_call("quest_decode"), flush, stream, args.steps)
        quest_separate = {}
        for name in ("quest_select_topk", "sparse_paged_attention_decode"):
            quest_separate[name] = time_alone(lambda: run_call(name), flush, stream,
                                              args.steps)["us_mean"]
        quest_separate["sum"] = round(sum(quest_separate.values()), 2)

    # The dense step as one call: the write (with the metadata fold when the step
    # keeps Quest metadata) merged into the dense decode call, timed alone behind the
    # flush. Idempotent like the step's own write.
    append_alone = quest_append_alone = None
    if w.num_tokens and w.num_tokens == B:
        append_alone = time_alone(lambda: gp.paged_attention_decode_append(
            q, nk, nv, kc, vc, slots, bt, ctx, max_context_len=mcl, scale=scale,
            key_min=kmin if fused else None, key_max=kmax if fused else None, out=out_d,
            workspace=ws_d), flush, stream, args.steps)
        if K:   # the Quest step as one call: the write folded into quest_decode
            quest_append_alone = time_alone(lambda: gp.quest_decode_append(
                q, nk, nv, kc, vc, kmin, kmax, slots, bt, ctx, topk_blocks=K, max_context_len=mcl,
                scale=scale, out=out_s, topk_out=sel, workspace=ws_qd), flush, stream, args.steps)

    # FP8 (E4M3) KV cache on the same workload: the pool quantised once by the FP8
    # write (every slot), then its write and dense calls timed like the bf16 ones.
    fp8 = None
    if not args.no_fp8:
        kc8, vc8, ks8, vs8 = fp8_copy(gp, kc, vc)
        out8 = torch.empty_like(out_d)
        fcalls = {
            "reshape_and_cache_fp8": lambda: gp.reshape_and_cache_fp8(nk, nv, kc8, vc8, ks8, vs8,
                                                                      slots),
            "paged_attention_decode_fp8": lambda: gp.paged_attention_decode_fp8(
                q, kc8, vc8, ks8, vs8, bt, ctx, max_context_len=mcl, scale=scale, out=out8,
                workspace=ws_d),
        }
        fbytes = {"reshape_and_cache_fp8": R.write_bytes(w.slot_mapping, w.num_blocks, bs, Hkv, D)
                  * 3 // 4,
                  "paged_attention_decode_fp8": R.dense_attention_bytes_fp8(w.context_lens, Hkv, D)}
        if w.num_tokens and w.num_tokens == B:   # the FP8 dense step as one call
            fcalls["paged_attention_decode_fp8_append"] = lambda: gp.paged_attention_decode_fp8_append(
                q, nk, nv, kc8, vc8, ks8, vs8, slots, bt, ctx, max_context_len=mcl, scale=scale,
                out=out8, workspace=ws_d)
            fbytes["paged_attention_decode_fp8_append"] = (fbytes["reshape_and_cache_fp8"]
                                                           + fbytes["paged_attention_decode_fp8"])
        if K:   # Quest over the E4M3 caches: code metadata built once (prefill work)
            kmin8 = torch.empty(kmin.shape, dtype=torch.uint8, device="cuda")
            kmax8 = torch.empty_like(kmin8)
            gp.quest_block_metadata_fp8(kc8, bt, ctx, kmin8, kmax8, max_context_len=mcl)
            sel8, out8s = torch.empty_like(sel), torch.empty_like(out_s)
            fcalls["quest_decode_fp8"] = lambda: gp.quest_decode_fp8(
                q, kc8, vc8, ks8, vs8, kmin8, kmax8, bt, ctx, topk_blocks=K, max_context_len=mcl,
                scale=scale, out=out8s, topk_out=sel8, workspace=ws_qd)
            fcalls["quest_decode_fp8"]()
            q8 = (R.select_bytes(w.context_lens, bs, Hkv, D, elem_bytes=1)
                  + R.sparse_attention_bytes(sel8.cpu().numpy(), w.context_lens, bs, D,
                                             elem_bytes=1))
            fbytes["quest_decode_fp8"] = q8
            if w.num_tokens and w.num_tokens == B:   # the FP8 Quest step as one call
                fcalls["quest_decode_fp8_append"] = lambda: gp.quest_decode_fp8_append(
                    q, nk, nv, kc8, vc8, ks8, vs8, kmin8, kmax8, slots, bt, ctx, topk_blocks=K,
                    max_context_len=mcl, scale=scale, out=out8s, topk_out=sel8, workspace=ws_qd)
                fbytes["quest_decode_fp8_append"] = q8 + R.fused_write_bytes_fp8(
                    w.slot_mapping, w.num_blocks, bs, Hkv, D)
        fp8 = {}
        for name, f in fcalls.items():
            for _ in range(3):
                f()
            ts = []
            for k in range(args.steps):
                flush.fill_(k & 0xFF)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                f()
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            t = float(np.mean(ts))
            fp8[name] = {"us_mean": round(t, 2), "algorithmic_bytes": int(fbytes[name]),
                         "gbps": round(fbytes[name] / (t * 1e-6) / 1e9, 1),
                         "pct_of_peak": round(100 * fbytes[name] / (t * 1e-6) / 1e9
                                              / R.MI355X_HBM_GBPS, 1)}
        del kc8, vc8
        if K:
            del kmin8, kmax8

    # Multi-token queries on the same caches: a mixed batch in which six sequences
    # bring prefill chunks (the newest positions of their contexts) and the rest
    # decode one token.
    varlen = None
    if not args.no_varlen and B >= 6:
        ql = np.ones(B, dtype=np.int64)
        ql[:6] = [128, 256, 64, 512, 32, 128]
        ql = np.minimum(ql, w.context_lens.astype(np.int64))
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(ql)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(12)
        qv = torch.randn((int(cu[-1]), Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
        cu_d = torch.from_numpy(cu).cuda()
        ws_v = torch.empty(gp.paged_attention_varlen_workspace_bytes(B, int(cu[-1]), int(ql.max()),
                                                                     Hq, Hkv, D, bs, mcl),
                           dtype=torch.uint8, device="cuda")
        out_v = torch.empty((int(cu[-1]), Hq, D), dtype=torch.float32, device="cuda")
        fv = lambda: gp.paged_attention_varlen(qv, kc, vc, bt, ctx, cu_d, max_q_len=int(ql.max()),
                                               max_context_len=mcl, scale=scale, out=out_v,
                                               workspace=ws_v)
        t = time_alone(fv, flush, stream, args.steps)["us_mean"]
        t8 = None
        if not args.no_fp8:   # the same batch over E4M3 copies of the caches
            kc8, vc8, ks8, vs8 = fp8_copy(gp, kc, vc)
            t8 = time_alone(lambda: gp.paged_attention_varlen_fp8(
                qv, kc8, vc8, ks8, vs8, bt, ctx, cu_d, max_q_len=int(ql.max()),
                max_context_len=mcl, scale=scale, out=out_v, workspace=ws_v),
                flush, stream, args.steps)["us_mean"]
            del kc8, vc8
        kv_bytes = R.dense_attention_bytes(w.context_lens, Hkv, D)
        ctx64 = w.context_lens.astype(np.int64)
        visible = int(sum(int((ctx64[b] - ql[b] + 1 + np.arange(ql[b])).sum()) for b in range(B)))
        flops = 4 * D * Hq * visible
        varlen = {"workload": "8K-average caches; q_len 128/256/64/512/32/128 for six sequences, "
                              "1 for the rest", "query_rows": int(cu[-1]), "us_mean": round(t, 2),
                  "kv_bytes_read_once": int(kv_bytes),
                  "gbps_kv_once": round(kv_bytes / (t * 1e-6) / 1e9, 1),
                  "tflops": round(flops / (t * 1e-6) / 1e12, 2),
                  "pct_of_8tbps": round(100 * kv_bytes / (t * 1e-6) / 1e9 / R.MI355X_HBM_GBPS, 1),
                  "pct_of_bf16_mfma_2500tflops": round(100 * flops / (t * 1e-6) / 1e12 / 2500.0, 2),
                  "fp8_kv_us_mean": round(t8, 2) if t8 else None}
        del qv, ws_v, out_v

    per_call = {name: np.array([evs[k][i].elapsed_time(evs[k][i + 1]) * 1e3 for k in range(args.steps)])
                for i, name in enumerate(calls)}
    step_us = np.array([evs[k][0].elapsed_time(evs[k][len(calls)]) * 1e3 for k in range(args.steps)])

    # Algorithmic bytes of one step.
    sel_host = sel.cpu().numpy() if K else None
    by = {
        "reshape_and_cache": R.write_bytes(w.slot_mapping, w.num_blocks, bs, Hkv, D),
        "reshape_and_cache_quest": R.fused_write_bytes(w.slot_mapping, w.num_blocks, bs, Hkv, D),
        "paged_attention_decode": R.dense_attention_bytes(w.context_lens, Hkv, D),
    }
    if K:
        by["quest_block_metadata"] = R.metadata_step_bytes(w.context_lens, bs, Hkv, D)
        by["quest_select_topk"] = R.select_bytes(w.context_lens, bs, Hkv, D)
        by["sparse_paged_attention_decode"] = R.sparse_attention_bytes(sel_host, w.context_lens, bs, D)
        by["quest_decode"] = by["quest_select_topk"] + by["sparse_paged_attention_decode"]
    # The one-call dense step: K / V of every valid token plus the write (with the
    # metadata fold when the step keeps Quest metadata).
    by["paged_attention_decode_append"] = by["paged_attention_decode"] + (
        by["reshape_and_cache_quest"] if K else by["reshape_and_cache"])
    step_bytes = sum(by[n] for n in calls)
    mean_step = float(step_us.mean())
    value = step_bytes / (mean_step * 1e-6) / 1e9

    calls_out = {}
    for name in calls:
        t = per_call[name]
        calls_out[name] = {
            "us_mean": round(float(t.mean()), 2), "us_median": round(float(np.median(t)), 2),
            "us_min": round(float(t.min()), 2), "algorithmic_bytes": int(by[name]),
            "gbps": round(by[name] / (t.mean() * 1e-6) / 1e9, 1) if by[name] else 0.0,
        }
        calls_out[name]["pct_of_peak"] = round(100 * calls_out[name]["gbps"] / R.MI355X_HBM_GBPS, 1)

    dense_t = per_call[dense_name].mean()
    achieved = by[dense_name] / (dense_t * 1e-6) / 1e9
    traffic = committed_traffic(args.config)
    # Both step figures include the write (when the workload has one): dense = write +
    # dense attention (one call on the append path); Quest = write (+ metadata refresh)
    # + the Quest part, which for the one-call path is quest_decode timed alone behind
    # its own flush (so it never follows the dense call's 1 GB stream), and on the
    # append path quest_decode_append timed alone (the write folded into it).
    write_us = sum(calls_out[n]["us_mean"] for n in calls
                   if n.startswith("reshape_and_cache"))
    if not K:
        quest_us = None
    elif one_call and write_mode == "append" and quest_append_alone:
        quest_us = quest_append_alone["us_mean"]
    elif one_call:
        quest_us = write_us + quest_alone["us_mean"]
    else:
        quest_us = sum(calls_out[n]["us_mean"] for n in calls if n != dense_name)

    line = {
        "metric": "paged decode attention KV-read HBM GB/s over one decode step (write + dense + Quest)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_step / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "global_batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": bs, "sum_context": int(w.context_lens.sum()),
                   "max_context_len": mcl, "topk_blocks": K, "parallelism": "single-gpu",
                   "write_path": write_mode if (K or write_mode == "append") else "plain",
                   "quest_path": ("one_call" if one_call else "separate") if K else None,
                   "sparse_split_tokens": gp.split_tokens(B, Hkv, K * bs) if K else None},
        "pct_of_peak": round(100 * value / R.MI355X_HBM_GBPS, 1),
        "us_per_step": round(mean_step, 2),
        "us_per_step_median": round(float(np.median(step_us)), 2),
        "dense_step_us": round(write_us + calls_out[dense_name]["us_mean"], 2),
        "dense_step_one_call": append_alone,
        "quest_step_one_call": quest_append_alone,
        "quest_step_us": round(quest_us, 2) if quest_us is not None else None,
        "quest_full_metadata_rebuild_us": round(t_full, 2) if t_full is not None else None,
        "graph_replay_us_per_step": round(graph_us, 2) if graph_us is not None else None,
        "fp8_kv": fp8,
        "varlen_mixed": varlen,
        "quest_decode_alone": quest_alone,
        "quest_separate_calls_us": quest_separate,
        "calls": calls_out,
        "step_algorithmic_bytes": int(step_bytes),
        "wall_s_timed_region_incl_flush": round(wall, 4),
        "flush_mib_between_steps": args.flush_mib,
        "roofline": {
            "bound": "hbm",
            "kernel": (f"{dense_name} call: {dominant_kernel(Hkv)} + its combine kernel"
                       + (" (which also writes the new tokens and folds them into the metadata)"
                          if dense_name.endswith("append") else "")),
            "achieved": round(achieved, 1), "peak": R.MI355X_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / R.MI355X_HBM_GBPS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": int(by[dense_name]),
            "launch_us_mean": round(float(dense_t), 2),
        },
        "kernel_source_sha256_16": kernel_source_hash(),
        "gpu": torch.cuda.get_device_name(0),
        "torch": torch.__version__, "hip": torch.version.hip,
    }
    if not args.no_per_config:
        del kc, vc, q, bt, ctx, nk, nv, slots, kmin, kmax, out_d, out_s, ws_d
        if K:
            del ws_sel, ws_sp, ws_qd, sel
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        blocks = {}
        for cfg in (1, 2, 3, 4, 5):
            print(f"[bench] per-workload block: config {cfg}", file=sys.stderr, flush=True)
            blocks[str(cfg)] = per_config_block(cfg, flush, stream, args.steps)
        line["per_config"] = blocks
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    if args.details:
        print(json.dumps(calls_out, indent=1), file=sys.stderr)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
