"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side argument checks return the documented status without launching."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from gqa_paged_kv_amd import _lib
    from gqa_paged_kv_amd import build as b
    srcs = [os.path.join(b.CSRC, s) for s in b.SOURCES] + \
        [os.path.join(b.CSRC, h) for h in os.listdir(b.CSRC) if h.endswith(".h")] + \
        [os.path.join(b.INCLUDE, "gpkv.h")]
    if not os.path.exists(_lib.LIB_PATH) or os.path.getmtime(_lib.LIB_PATH) < max(map(os.path.getmtime, srcs)):
        b.build()
    return _lib.lib()


def declared_symbols():
    with open(os.path.join(ROOT, "include", "gpkv.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(gpkv_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    from gqa_paged_kv_amd._lib import SIGNATURES
    names = declared_symbols()
    assert len(names) == 29
    for n in names:
        assert hasattr(L, n), n
    assert sorted(SIGNATURES) == names


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5):
        assert L.gpkv_status_string(st)
    assert L.gpkv_status_string(7) == b"unknown status"


ARGS = dict(B=2, Hq=4, Hkv=1, D=64, bs=16, NB=16, MB=5, mcl=80)


def _dense(L, **o):
    a = {**ARGS, **o}
    ws = o.get("ws", 1 << 40)
    return L.gpkv_paged_attention_decode(
        o.get("out", 8), 8, 8, 8, 8, 8, a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"],
        a["MB"], a["mcl"], 0.125, o.get("wsp", 8), ws, None)


@pytest.mark.parametrize("override,status", [
    (dict(out=None), -1),
    (dict(Hq=6, Hkv=4), -2),
    (dict(Hq=34, Hkv=2), -3),       # group 17 > 16
    (dict(D=96), -3),
    (dict(bs=8), -3),
    (dict(bs=24), -3),
    (dict(mcl=81), -2),             # > max_blocks * block_size
    (dict(B=-1), -2),
    (dict(ws=16), -4),
    (dict(wsp=None), -4),
])
def test_dense_argument_checks(L, override, status):
    assert _dense(L, **override) == status
    assert L.gpkv_last_error_message()


def test_other_entry_points_checks(L):
    # reshape_and_cache: null pointers, bad head_dim; zero tokens is a no-op.
    assert L.gpkv_reshape_and_cache(None, 8, 8, 8, 8, 2, 1, 64, 16, 16, None) == -1
    assert L.gpkv_reshape_and_cache(8, 8, 8, 8, 8, 2, 1, 80, 16, 16, None) == -3
    assert L.gpkv_reshape_and_cache(None, None, None, None, None, 0, 1, 64, 16, 16, None) == 0
    # metadata
    assert L.gpkv_quest_block_metadata(None, 8, 8, 8, 8, 2, 1, 64, 16, 16, 5, 80, 0, None) == -1
    assert L.gpkv_quest_block_metadata(8, 8, 8, 8, 8, 2, 1, 64, 16, 16, 4, 80, 0, None) == -2
    # top-k: topk_blocks < 1, workspace too small, group too large
    assert L.gpkv_quest_select_topk(8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 0, 8, 1 << 30, None) == -2
    assert L.gpkv_quest_select_topk(8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 3, 8, 8, None) == -4
    assert L.gpkv_quest_select_topk(8, 8, 8, 8, 8, 8, 2, 40, 2, 64, 16, 16, 5, 80, 3, 8, 1 << 30, None) == -3
    # sparse: null topk, topk_blocks < 1
    assert L.gpkv_sparse_paged_attention_decode(8, 8, 8, 8, 8, 8, None, 2, 4, 1, 64, 16, 16, 5, 80, 3,
                                                0.1, 8, 1 << 30, None) == -1
    assert L.gpkv_sparse_paged_attention_decode(8, 8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 0,
                                                0.1, 8, 1 << 30, None) == -2
    # fused write: null metadata, bad block size; zero tokens is a no-op
    assert L.gpkv_reshape_and_cache_quest(8, 8, 8, 8, None, 8, 8, 2, 1, 64, 16, 16, None) == -1
    assert L.gpkv_reshape_and_cache_quest(8, 8, 8, 8, 8, 8, 8, 2, 1, 64, 24, 16, None) == -3
    assert L.gpkv_reshape_and_cache_quest(None, None, None, None, None, None, None, 0, 1, 64, 16,
                                          16, None) == 0
    # FP8 write: null scale, bad head_dim, zero tokens
    assert L.gpkv_reshape_and_cache_fp8(8, 8, 8, 8, None, 8, 8, 2, 1, 64, 16, 16, None) == -1
    assert L.gpkv_reshape_and_cache_fp8(8, 8, 8, 8, 8, 8, 8, 2, 1, 96, 16, 16, None) == -3
    assert L.gpkv_reshape_and_cache_fp8(None, None, None, None, None, None, None, 0, 1, 64, 16, 16,
                                        None) == 0
    # FP8 attention: null scales, small workspace; sparse FP8: null list
    assert L.gpkv_paged_attention_decode_fp8(8, 8, 8, 8, None, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80,
                                             0.1, 8, 1 << 30, None) == -1
    assert L.gpkv_paged_attention_decode_fp8(8, 8, 8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80,
                                             0.1, 8, 16, None) == -4
    assert L.gpkv_sparse_paged_attention_decode_fp8(8, 8, 8, 8, 8, 8, 8, 8, None, 2, 4, 1, 64, 16,
                                                    16, 5, 80, 3, 0.1, 8, 1 << 30, None) == -1
    # varlen: null cu_seqlens, zero rows is a no-op, max_q_len 0 with rows, small workspace
    assert L.gpkv_paged_attention_varlen(8, 8, 8, 8, 8, 8, None, 2, 5, 4, 4, 1, 64, 16, 16, 5, 80,
                                         0.1, 8, 1 << 30, None) == -1
    assert L.gpkv_paged_attention_varlen(None, None, None, None, None, None, None, 2, 0, 4, 4, 1,
                                         64, 16, 16, 5, 80, 0.1, None, 0, None) == 0
    assert L.gpkv_paged_attention_varlen(8, 8, 8, 8, 8, 8, 8, 2, 5, 0, 4, 1, 64, 16, 16, 5, 80,
                                         0.1, 8, 1 << 30, None) == -2
    assert L.gpkv_paged_attention_varlen(8, 8, 8, 8, 8, 8, 8, 2, 5, 4, 4, 1, 64, 16, 16, 5, 80,
                                         0.1, 8, 16, None) == -4
    assert L.gpkv_paged_attention_varlen_workspace_bytes(2, 5, 4, 4, 1, 64, 16, 80) > 0
    # FP8 varlen: null scales, small workspace
    assert L.gpkv_paged_attention_varlen_fp8(8, 8, 8, 8, None, 8, 8, 8, 8, 2, 5, 4, 4, 1, 64, 16,
                                             16, 5, 80, 0.1, 8, 1 << 30, None) == -1
    assert L.gpkv_paged_attention_varlen_fp8(8, 8, 8, 8, 8, 8, 8, 8, 8, 2, 5, 4, 4, 1, 64, 16, 16,
                                             5, 80, 0.1, 8, 16, None) == -4
    # one-call Quest decode: null selection output, topk_blocks < 1, small workspace
    assert L.gpkv_quest_decode(8, None, 8, 8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 3, 0.1, 8,
                               1 << 30, None) == -1
    assert L.gpkv_quest_decode(8, 8, 8, 8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 0, 0.1, 8,
                               1 << 30, None) == -2
    assert L.gpkv_quest_decode(8, 8, 8, 8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 3, 0.1, 8,
                               16, None) == -4
    assert L.gpkv_quest_decode_workspace_bytes(2, 4, 1, 64, 16, 5, 3) >= max(
        L.gpkv_quest_select_workspace_bytes(2, 1, 5),
        L.gpkv_sparse_attention_workspace_bytes(2, 4, 1, 64, 16, 3))


def test_append_argument_checks(L):
    """The dense call with the step's cache write: its own pointers (new rows, slots,
    metadata given as a pair) and the dense call's checks, all refused on the host
    (no call here launches anything)."""
    a = ARGS
    f = L.gpkv_paged_attention_decode_append

    def call(key=8, kmin=None, kmax=None, slots=8, ws=1 << 40, D=a["D"], B=a["B"], wsp=8):
        return f(8, 8, key, 8, 8, 8, kmin, kmax, slots, 8, 8, B, a["Hq"], a["Hkv"], D, a["bs"],
                 a["NB"], a["MB"], a["mcl"], 0.125, wsp, ws, None)

    assert call(key=None) == -1
    assert call(slots=None) == -1
    assert call(kmin=8) == -1          # key_min without key_max
    assert call(kmax=8) == -1
    assert call(D=96) == -3
    assert call(ws=16) == -4
    assert call(B=0, key=None, slots=None) == 0   # an empty batch launches nothing
    # the FP8 form: scales required as for the FP8 dense call
    g = L.gpkv_paged_attention_decode_fp8_append
    base = [8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"],
            a["MB"], a["mcl"], 0.125, 8, 1 << 40, None]
    for i in (2, 3, 6, 7, 8):   # key, value, k_scale, v_scale, slot_mapping
        args = list(base)
        args[i] = None
        assert g(*args) == -1, i
    args = list(base)
    args[21] = 16
    assert g(*args) == -4


def test_quest_append_argument_checks(L):
    """The Quest step with its cache write: new rows and slots required, topk_blocks
    and the workspace checked like quest_decode, all refused on the host."""
    f = L.gpkv_quest_decode_append

    def call(key=8, slots=8, K=3, ws=1 << 30, B=2):
        return f(8, 8, 8, key, 8, 8, 8, 8, 8, slots, 8, 8, B, 4, 1, 64, 16, 16, 5, 80, K, 0.1, 8,
                 ws, None)

    assert call(key=None) == -1
    assert call(slots=None) == -1
    assert call(K=0) == -2
    assert call(ws=16) == -4
    assert call(B=0, key=None, slots=None) == 0


def test_quest_fp8_argument_checks(L):
    """Quest over E4M3 caches: scales and metadata required, shapes and sizes checked as
    for the bf16 calls, all refused on the host (an empty batch launches nothing)."""
    m = L.gpkv_quest_block_metadata_fp8
    assert m(None, 8, 8, 8, 8, 2, 1, 64, 16, 16, 5, 80, 0, None) == -1
    assert m(8, 8, 8, 8, 8, 2, 1, 96, 16, 16, 5, 80, 0, None) == -3
    assert m(8, 8, 8, 8, 8, 2, 1, 64, 16, 16, 5, 81, 0, None) == -2    # past the table
    assert m(None, None, None, None, None, 0, 1, 64, 16, 16, 5, 80, 0, None) == 0
    w = L.gpkv_reshape_and_cache_fp8_quest
    assert w(8, 8, 8, 8, None, 8, 8, 8, 8, 2, 1, 64, 16, 16, None) == -1    # k_scale
    assert w(8, 8, 8, 8, 8, 8, None, 8, 8, 2, 1, 64, 16, 16, None) == -1    # key_min
    assert w(8, 8, 8, 8, 8, 8, 8, 8, 8, 2, 1, 64, 24, 16, None) == -3
    assert w(None, None, None, None, None, None, None, None, None, 0, 1, 64, 16, 16, None) == 0
    t = L.gpkv_quest_select_topk_fp8
    assert t(8, 8, None, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 3, 8, 1 << 30, None) == -1
    assert t(8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 0, 8, 1 << 30, None) == -2
    assert t(8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 3, 8, 8, None) == -4
    d = L.gpkv_quest_decode_fp8
    base = [8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 3, 0.1, 8, 1 << 30, None]
    for i in (1, 5, 6, 7, 8):          # topk_out, k_scale, v_scale, key_min, key_max
        args = list(base)
        args[i] = None
        assert d(*args) == -1, i
    args = list(base)
    args[19] = 0
    assert d(*args) == -2
    args = list(base)
    args[22] = 16
    assert d(*args) == -4
    a = L.gpkv_quest_decode_fp8_append
    base = [8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, 2, 4, 1, 64, 16, 16, 5, 80, 3, 0.1, 8,
            1 << 30, None]
    for i in (3, 4, 7, 8, 11):         # key, value, k_scale, v_scale, slot_mapping
        args = list(base)
        args[i] = None
        assert a(*args) == -1, i
    args = list(base)
    args[25] = 16
    assert a(*args) == -4
    args = list(base)
    args[14] = 0
    args[3] = args[11] = None
    assert a(*args) == 0


def test_noalloc_argument_checks(L):
    """The allocation-free dense call: null pointers, shapes, and sizes whose partial
    rows would not fit the library's 32 MiB device array are refused on the host."""
    a = ARGS
    base = [8, 8, 8, 8, 8, 8, a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["MB"], a["mcl"],
            0.125, None]
    f = L.gpkv_paged_attention_decode_noalloc
    assert f(*([None] + base[1:])) == -1
    bad = list(base)
    bad[13] = 81                      # max_context_len > max_blocks * block_size
    assert f(*bad) == -2
    big = [8, 8, 8, 8, 8, 8, 4096, 64, 8, 128, 16, 1 << 20, 2048, 32768, 0.1, None]
    assert L.gpkv_paged_attention_workspace_bytes(4096, 64, 8, 128, 16, 32768) > 32 << 20
    assert f(*big) == -4
    assert b"32" in L.gpkv_last_error_message() or b"scratch" in L.gpkv_last_error_message()
    zero = list(base)
    zero[6] = 0                        # an empty batch is a no-op
    assert f(*zero) == 0


def test_workspace_queries(L):
    assert L.gpkv_paged_attention_workspace_bytes(2, 4, 1, 64, 16, 80) > 0
    assert L.gpkv_paged_attention_workspace_bytes(2, 4, 1, 96, 16, 80) == 0
    assert L.gpkv_sparse_attention_workspace_bytes(2, 4, 1, 64, 16, 0) == 0
    assert L.gpkv_quest_select_workspace_bytes(64, 4, 1024) == 64 * 4 * 1024 * 8
    # split size: a multiple of 128 in [128, 1024]; enough units for the 8K-average workload
    t = L.gpkv_split_tokens(64, 4, 14998)
    assert t % 128 == 0 and 128 <= t <= 1024
    assert 64 * 4 * -(-14998 // t) >= 4096
