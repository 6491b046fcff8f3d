"""Byte accounting pinned to the worked numbers of the TileLang tutorial's KV ledger."""
import json
import os

import numpy as np

from gqa_paged_kv_amd import roofline as R

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kv_ledger_tl18.json")


def test_kv_ledger_matches_tutorial():
    g = json.load(open(GOLD))
    m = g["model"]
    per = R.kv_bytes_per_token_layer(m["num_kv_heads"], m["head_dim"], m["elem_bytes"])
    assert per == g["bytes_per_token_per_layer"]
    assert per * m["layers"] == g["bytes_per_token_all_layers"]
    assert per * m["layers"] * 16 == g["kib_per_16_token_block_all_layers"] * 1024
    assert per * m["layers"] * 131072 == g["gib_per_131072_token_sequence_all_layers"] * 2**30
    mha = R.kv_bytes_per_token_layer(m["num_q_heads"], m["head_dim"], m["elem_bytes"])
    assert mha * m["layers"] * 131072 == g["gib_per_131072_token_sequence_all_layers_mha"] * 2**30
    # one decode step at b=1, ctx=8192 reads the whole cache of every layer once
    dense = R.dense_attention_bytes([8192], m["num_kv_heads"], m["head_dim"]) * m["layers"]
    assert dense == g["mib_kv_traffic_b1_ctx8192_all_layers"] * 2**20
    assert R.decode_attention_ai(m["num_q_heads"], m["num_kv_heads"]) == g["decode_attention_ai_flop_per_byte"]


def test_sparse_and_metadata_accounting_by_hand():
    # ctx 37, bs 16: blocks 0, 1 full, block 2 holds 5 tokens; H_kv 1, D 64
    sel = np.array([[[0, 2, -1]]])
    assert R.sparse_attention_bytes(sel, [37], 16, 64) == (16 + 5) * 2 * 64 * 2
    assert R.metadata_step_bytes([37, 32], 16, 1, 64) == (5 + 16) * 128 + 2 * 2 * 128
    assert R.select_bytes([37, 32], 16, 1, 64) == (3 + 2) * 2 * 64 * 2
    assert R.write_bytes([5, -1, 10**9], 16, 16, 1, 64) == 1 * 2 * 64 * 2 * 2
    # slot 5 folds into its block (row 5), slot 32 starts a block (row 0)
    assert R.fused_write_bytes([5, 32, -1], 16, 16, 1, 64) == 2 * 4 * 128 + 1 * 2 * 128 + 2 * 2 * 128


def test_fp8_quest_accounting_by_hand():
    # one byte per element: the selection's metadata scan and the sparse K / V halve
    sel = np.array([[[0, 2, -1]]])
    assert R.sparse_attention_bytes(sel, [37], 16, 64, elem_bytes=1) == (16 + 5) * 2 * 64
    assert R.select_bytes([37, 32], 16, 1, 64, elem_bytes=1) == (3 + 2) * 2 * 64
    # H_kv 1, D 64: per token bf16 K and V in (2 * 128 bytes), codes out (2 * 64);
    # slot 5 folds (reads its block's two 64-byte code rows), both write two
    assert R.fused_write_bytes_fp8([5, 32, -1], 16, 16, 1, 64) == \
        2 * (2 * 128 + 2 * 64) + 1 * 2 * 64 + 2 * 2 * 64
