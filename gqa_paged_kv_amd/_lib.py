"""ctypes loader for libgpkv.so (argument marshalling only).

The library is built in-tree by ``python -m gqa_paged_kv_amd.build``. There is no
fallback: if the shared object is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgpkv.so")

c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_size = ctypes.c_size_t
c_float = ctypes.c_float
vp = ctypes.c_void_p

# name -> (restype, argtypes), in the order of include/gpkv.h
SIGNATURES = {
    "gpkv_reshape_and_cache": (c_int32, [vp, vp, vp, vp, vp, c_int32, c_int32, c_int32, c_int32,
                                         c_int64, vp]),
    "gpkv_reshape_and_cache_quest": (c_int32, [vp, vp, vp, vp, vp, vp, vp, c_int32, c_int32,
                                               c_int32, c_int32, c_int64, vp]),
    "gpkv_paged_attention_workspace_bytes": (c_size, [c_int32] * 6),
    "gpkv_paged_attention_decode": (c_int32, [vp, vp, vp, vp, vp, vp, c_int32, c_int32, c_int32,
                                              c_int32, c_int32, c_int64, c_int32, c_int32,
                                              c_float, vp, c_size, vp]),
    "gpkv_paged_attention_decode_append": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                     c_int32, c_int32, c_int32, c_int32, c_int32,
                                                     c_int64, c_int32, c_int32, c_float, vp,
                                                     c_size, vp]),
    "gpkv_paged_attention_decode_noalloc": (c_int32, [vp, vp, vp, vp, vp, vp, c_int32, c_int32,
                                                      c_int32, c_int32, c_int32, c_int64, c_int32,
                                                      c_int32, c_float, vp]),
    "gpkv_quest_block_metadata": (c_int32, [vp, vp, vp, vp, vp, c_int32, c_int32, c_int32,
                                            c_int32, c_int64, c_int32, c_int32, c_int32, vp]),
    "gpkv_quest_select_workspace_bytes": (c_size, [c_int32] * 3),
    "gpkv_quest_select_topk": (c_int32, [vp, vp, vp, vp, vp, vp, c_int32, c_int32, c_int32,
                                         c_int32, c_int32, c_int64, c_int32, c_int32, c_int32,
                                         vp, c_size, vp]),
    "gpkv_sparse_attention_workspace_bytes": (c_size, [c_int32] * 6),
    "gpkv_sparse_paged_attention_decode": (c_int32, [vp, vp, vp, vp, vp, vp, vp, c_int32,
                                                     c_int32, c_int32, c_int32, c_int32,
                                                     c_int64, c_int32, c_int32, c_int32,
                                                     c_float, vp, c_size, vp]),
    "gpkv_quest_decode_workspace_bytes": (c_size, [c_int32] * 7),
    "gpkv_quest_decode": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int32, c_int32,
                                    c_int32, c_int32, c_int32, c_int64, c_int32, c_int32,
                                    c_int32, c_float, vp, c_size, vp]),
    "gpkv_quest_decode_append": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           c_int32, c_int32, c_int32, c_int32, c_int32, c_int64,
                                           c_int32, c_int32, c_int32, c_float, vp, c_size, vp]),
    "gpkv_reshape_and_cache_fp8": (c_int32, [vp, vp, vp, vp, vp, vp, vp, c_int32, c_int32,
                                             c_int32, c_int32, c_int64, vp]),
    "gpkv_paged_attention_decode_fp8": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, c_int32,
                                                  c_int32, c_int32, c_int32, c_int32, c_int64,
                                                  c_int32, c_int32, c_float, vp, c_size, vp]),
    "gpkv_paged_attention_decode_fp8_append": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                         vp, c_int32, c_int32, c_int32, c_int32,
                                                         c_int32, c_int64, c_int32, c_int32,
                                                         c_float, vp, c_size, vp]),
    "gpkv_sparse_paged_attention_decode_fp8": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                         c_int32, c_int32, c_int32, c_int32,
                                                         c_int32, c_int64, c_int32, c_int32,
                                                         c_int32, c_float, vp, c_size, vp]),
    "gpkv_quest_block_metadata_fp8": (c_int32, [vp, vp, vp, vp, vp, c_int32, c_int32, c_int32,
                                                c_int32, c_int64, c_int32, c_int32, c_int32, vp]),
    "gpkv_reshape_and_cache_fp8_quest": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int32,
                                                   c_int32, c_int32, c_int32, c_int64, vp]),
    "gpkv_quest_select_topk_fp8": (c_int32, [vp, vp, vp, vp, vp, vp, c_int32, c_int32, c_int32,
                                             c_int32, c_int32, c_int64, c_int32, c_int32, c_int32,
                                             vp, c_size, vp]),
    "gpkv_quest_decode_fp8": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int32,
                                        c_int32, c_int32, c_int32, c_int32, c_int64, c_int32,
                                        c_int32, c_int32, c_float, vp, c_size, vp]),
    "gpkv_quest_decode_fp8_append": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, c_int32, c_int32, c_int32, c_int32, c_int32,
                                               c_int64, c_int32, c_int32, c_int32, c_float, vp,
                                               c_size, vp]),
    "gpkv_paged_attention_varlen_workspace_bytes": (c_size, [c_int32] * 8),
    "gpkv_paged_attention_varlen": (c_int32, [vp, vp, vp, vp, vp, vp, vp, c_int32, c_int32,
                                              c_int32, c_int32, c_int32, c_int32, c_int32,
                                              c_int64, c_int32, c_int32, c_float, vp, c_size,
                                              vp]),
    "gpkv_paged_attention_varlen_fp8": (c_int32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int32,
                                                  c_int32, c_int32, c_int32, c_int32, c_int32,
                                                  c_int32, c_int64, c_int32, c_int32, c_float,
                                                  vp, c_size, vp]),
    "gpkv_status_string": (ctypes.c_char_p, [c_int32]),
    "gpkv_last_error_message": (ctypes.c_char_p, []),
    "gpkv_split_tokens": (c_int32, [c_int32, c_int32, c_int32]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libgpkv.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m gqa_paged_kv_amd.build` first")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib
