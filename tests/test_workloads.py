"""The seeded input generators: bf16 rounding, the recipes, and the Top-K tie guard."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 np.float32)])
    ours = workloads.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("config", [1, 2, 4])
def test_recipe_shapes_and_tables(config):
    w = workloads.make(config)
    B, bs = w.batch, w.block_size
    assert w.key_cache.shape == (w.num_blocks, bs, w.num_kv_heads, w.head_dim)
    assert w.query.shape == (B, w.num_q_heads, w.head_dim)
    nb = w.nblocks()
    used = np.concatenate([w.block_tables[b, :nb[b]] for b in range(B)])
    assert len(np.unique(used)) == used.size, "a physical block is shared"
    assert used.min() >= 0 and used.max() < w.num_blocks
    assert (w.block_tables[np.arange(w.max_blocks_per_seq)[None, :] >= nb[:, None]] == -1).all()
    assert w.max_context_len <= w.max_blocks_per_seq * bs
    for i, s in enumerate(w.slot_mapping.tolist()):
        if s >= 0:   # the new token sits at its sequence's last position
            assert any(s == int(w.block_tables[b, (int(w.context_lens[b]) - 1) // bs]) * bs
                       + (int(w.context_lens[b]) - 1) % bs for b in range(B))
    assert w.scale == np.float32(1 / math.sqrt(w.head_dim))


def test_config_specifics():
    w1 = workloads.make(1)
    assert w1.context_lens.tolist() == [37, 80] and w1.slot_mapping[1] == -1
    w4 = workloads.make(4)
    assert (w4.context_lens == 40960).all() and w4.num_blocks == 10240


def _min_relative_gap(w, K):
    """Smallest gap between the K-th and (K+1)-th score over all (b, g), relative."""
    kmin, kmax = oracle.quest_block_metadata(w.key_cache, w.block_tables, w.context_lens,
                                             w.block_size)
    worst = np.inf
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            s = oracle.quest_block_scores(w.query, kmin, kmax, w.block_tables, w.context_lens,
                                          w.block_size, b, g)
            if s.size <= K:
                continue
            top = np.sort(s)[::-1]
            gap = (top[K - 1] - top[K]) / max(abs(top[K - 1]), 1e-300)
            worst = min(worst, gap)
    return worst


@pytest.mark.parametrize("config", [1, 3, 4, 5])
def test_topk_has_no_near_ties(config):
    """Float64 on the GPU and fsum in the oracle agree on the selection only when the
    K-th and (K+1)-th scores are well apart; the seeded configs must keep them apart."""
    w = workloads.make(config)
    for K in w.topk_list:
        gap = _min_relative_gap(w, K)
        assert gap > 1e-9, f"config {config} K={K}: near-tie, relative gap {gap:.3e}"


def _fp8_min_relative_gap(w, K):
    """The same gap for Quest over E4M3 caches: codes made with the per-head scales the
    GPU tests use (amax of a fixed subsample / 256), code metadata, scores on codes."""
    from gpu_util import fp8_codes
    from test_fp8_gpu import _scales
    kc = fp8_codes(w.key_cache, _scales(w.key_cache))
    kmin, kmax = oracle.quest_block_metadata_fp8(kc, w.block_tables, w.context_lens,
                                                 w.block_size)
    worst = np.inf
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            s = oracle.quest_block_scores_fp8(w.query, kmin, kmax, w.block_tables,
                                              w.context_lens, w.block_size, b, g)
            if s.size <= K:
                continue
            top = np.sort(s)[::-1]
            gap = (top[K - 1] - top[K]) / max(abs(top[K - 1]), 1e-300)
            worst = min(worst, gap)
    return worst


@pytest.mark.parametrize("config", [1, 3, 4, 5])
def test_fp8_topk_has_no_near_ties(config):
    """The FP8 selections the GPU tests compare bit for bit are just as well separated."""
    w = workloads.make(config)
    for K in w.topk_list:
        gap = _fp8_min_relative_gap(w, K)
        assert gap > 1e-9, f"config {config} K={K}: near-tie, relative gap {gap:.3e}"
