"""Dense decode without allocation (gpkv_paged_attention_decode_noalloc): its partial
rows live in the library's fixed device array instead of a caller workspace.

Two calls in a row on one GPU, the second smaller than the first, each against the
call that takes a workspace (bit for bit: the same kernels and work split) and
against the oracle (max-abs 2e-3); sizes past the array are refused.
"""
import numpy as np
import pytest
import torch

import gqa_paged_kv_amd as gp
import oracle
import workloads
from gpu_util import Dev, dense_ref, max_abs, workload

pytestmark = pytest.mark.gpu
ATOL = 2e-3


def _both(w):
    d = Dev(w)
    if w.num_tokens:   # the step writes the new token first (context_lens include it)
        gp.reshape_and_cache(d.nk, d.nv, d.kc, d.vc, d.slots)
    shape = (w.batch, w.num_q_heads, w.head_dim)
    out_n = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    gp.paged_attention_decode_noalloc(d.q, d.kc, d.vc, d.bt, d.ctx, out_n,
                                      max_context_len=w.max_context_len, scale=float(w.scale))
    out_w = gp.paged_attention_decode(d.q, d.kc, d.vc, d.bt, d.ctx,
                                      max_context_len=w.max_context_len, scale=float(w.scale))
    torch.cuda.synchronize()
    return out_n, out_w


def test_noalloc_two_calls_equal_workspace_call_and_oracle():
    big = workload(5)            # ragged 256-sequence batch, 8 KV heads: ~16 MiB of partials
    need = gp.paged_attention_workspace_bytes(big.batch, big.num_q_heads, big.num_kv_heads,
                                              big.head_dim, big.block_size, big.max_context_len)
    assert 8 << 20 < need <= 32 << 20
    small = workloads.random_case(951, batch=5, num_q_heads=16, num_kv_heads=2, head_dim=64,
                                  block_size=32, context_lens=[0, 1, 700, 33, 2100])
    for w, ref in ((big, lambda: dense_ref(5)),
                   (small, lambda: oracle.paged_attention_decode(
                       small.query, small.key_cache, small.value_cache, small.block_tables,
                       small.context_lens, small.scale))):
        out_n, out_w = _both(w)
        assert torch.equal(out_n, out_w), "no-alloc call differs from the workspace call"
        err = max_abs(out_n.cpu().numpy(), ref())
        print(f"{w.name}: no-alloc max-abs vs oracle {err:.3e}")
        assert err <= ATOL


def test_noalloc_refuses_sizes_past_the_array():
    w = workloads.random_case(952, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                              block_size=16, context_lens=[40, 17])
    d = Dev(w)
    B = 4096
    q = torch.zeros((B, 64, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 2048), dtype=torch.int32, device="cuda")
    ctx = torch.zeros((B,), dtype=torch.int32, device="cuda")
    kc = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, 64, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(gp.GpkvError) as exc:
        gp.paged_attention_decode_noalloc(q, kc, kc, bt, ctx, out, max_context_len=32768,
                                          scale=0.1)
    assert exc.value.status == -4
    out2 = torch.zeros((2, 8, 128), dtype=torch.float32, device="cuda")
    gp.paged_attention_decode_noalloc(d.q, d.kc, d.vc, d.bt, d.ctx, out2,
                                      max_context_len=w.max_context_len, scale=float(w.scale))
    torch.cuda.synchronize()
    ref = oracle.paged_attention_decode(w.query, w.key_cache, w.value_cache, w.block_tables,
                                        w.context_lens, w.scale)
    assert max_abs(out2.cpu().numpy(), ref) <= ATOL
