"""Plant plausible mistakes in copies of the oracle and check the pins catch each.

Each mutant is a one-line textual change to oracle/__init__.py, executed as a
fresh module on the CPU. A mutant survives only if every pin still passes; the
test fails on a survivor, which would mean the pins cannot see that mistake.
"""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "__init__.py")

MUTANTS = [
    ("write: block/offset swapped", "blk, off = divmod(s, block_size)", "off, blk = divmod(s, block_size)"),
    ("write: slot 0 skipped", "        if s < 0:\n            continue", "        if s <= 0:\n            continue"),
    ("write: key row into value cache", "vc[blk, off] = value[i]", "vc[blk, off] = key[i]"),
    ("dense: scale dropped", "sc = float(np.float32(scale))", "sc = 1.0"),
    ("dense: interleaved head groups", "heads = slice(g * G, (g + 1) * G)\n            out[b, heads] = _softmax_attention(q[b, heads], k[:, g]",
     "heads = slice(g, Hq, Hkv)\n            out[b, heads] = _softmax_attention(q[b, heads], k[:, g]"),
    ("dense: last token dropped", "pos = np.arange(int(ctx[b]))", "pos = np.arange(max(int(ctx[b]) - 1, 0))"),
    ("gather: row offset off by one", "return cache_f64[pb, pos % block_size]", "return cache_f64[pb, (pos + 1) % block_size]"),
    ("softmax: no normalisation", "p = e / e.sum(axis=1, keepdims=True)", "p = e"),
    ("softmax: K used as V", "    return p @ v\n", "    return p @ k\n"),
    ("combine: unit weights", "w = np.exp(lses - safe)", "w = np.where(np.isfinite(lses), 1.0, 0.0)"),
    ("meta: invalid tokens included", "n = min(bs, L - lb * bs)\n            k = bf16_to_f64", "n = bs\n            k = bf16_to_f64"),
    ("meta: min and max swapped", "kmin[pb] = f64_to_bf16_exact(k.min(axis=0))", "kmin[pb] = f64_to_bf16_exact(k.max(axis=0))"),
    ("meta: step mode updates block 0", "blocks = [nb - 1] if", "blocks = [0] if"),
    ("score: min instead of max", "terms = np.maximum(", "terms = np.minimum("),
    ("score: wrong query group", "q = bf16_to_f64(query[b, g * G:(g + 1) * G])", "q = bf16_to_f64(query[b, g:g + G])"),
    ("score: kmin used for both bounds", "hi = bf16_to_f64(key_max[pbs, g])", "hi = bf16_to_f64(key_min[pbs, g])"),
    ("topk: ties to the higher index", "key=lambda lb: (-s[lb], lb)", "key=lambda lb: (-s[lb], -lb)"),
    ("topk: output not ascending", "keep = sorted(order[:min(topk, s.size)])", "keep = order[:min(topk, s.size)]"),
    ("topk: ascending score order", "key=lambda lb: (-s[lb], lb)", "key=lambda lb: (s[lb], lb)"),
    ("sparse: block 0 never attended", "if x >= 0})", "if x > 0})"),
    ("sparse: last block not masked", "pos.extend(range(lb * block_size, min((lb + 1) * block_size, int(ctx))))",
     "pos.extend(range(lb * block_size, (lb + 1) * block_size))"),
    ("sparse: selection of KV head 0 for all", "pos = sparse_token_positions(topk_indices[b, g], ctx[b], bs)",
     "pos = sparse_token_positions(topk_indices[b, 0], ctx[b], bs)"),
    ("fp8: ties away from zero", "np.where(lo % 2 == 0, lo, hi)", "hi"),
    ("fp8: exponent bias 8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("fp8: subnormal step 2^-8", "m * 2.0 ** -9", "m * 2.0 ** -8"),
    ("fp8: sign dropped on encode",
     "code = pick.astype(np.uint8) | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))",
     "code = pick.astype(np.uint8)"),
    ("fp8: scale multiplied on write", "y = (x * inv[:, None])",
     "y = (x * np.asarray(scale, dtype=np.float32)[:, None])"),
    ("fp8: k scale dropped on read", "* ks[:, None]", "* 1.0"),
    ("fp8: v scale dropped on read", "* vs[:, None]", "* 1.0"),
    ("varlen: mask aligned left", "lim = L - (r1 - r0) + np.arange(r1 - r0)", "lim = np.arange(r1 - r0)"),
    ("varlen: mask off by one", "visible = pos[None, :] <= lim[:, None]", "visible = pos[None, :] < lim[:, None]"),
    ("varlen: no causal mask", "visible = pos[None, :] <= lim[:, None]", "visible = pos[None, :] >= 0"),
    ("fp8 varlen: K scale on V", "                e4m3_to_f64(gather_sequence(value_cache, block_tables, b, pos, bs)) * vs[:, None])",
     "                e4m3_to_f64(gather_sequence(value_cache, block_tables, b, pos, bs)) * ks[:, None])"),
    ("fp8 varlen: codes read as bf16", "        return (e4m3_to_f64(gather_sequence(key_cache, block_tables, b, pos, bs)) * ks[:, None],",
     "        return (bf16_to_f64(gather_sequence(key_cache, block_tables, b, pos, bs)) * ks[:, None],"),
    ("fp8 sparse: K scale on V", "* vs[g]", "* ks[g]"),
    ("fp8 sparse: KV head 0's keys for every head",
     "k_g = e4m3_to_f64(gather_sequence(key_cache[:, :, g]", "k_g = e4m3_to_f64(gather_sequence(key_cache[:, :, 0]"),
    ("fp8 sparse: no K scale", "key_cache[:, :, g], block_tables, b, pos, bs)) * ks[g]",
     "key_cache[:, :, g], block_tables, b, pos, bs))"),
    ("fp8 meta: invalid rows included", "n = min(bs, L - lb * bs)\n            k = e4m3_to_f64",
     "n = bs\n            k = e4m3_to_f64"),
    ("fp8 meta: min and max swapped", "kmin[pb] = e4m3_code_of(k.min(axis=0))",
     "kmin[pb] = e4m3_code_of(k.max(axis=0))"),
    ("fp8 meta: step mode updates block 0",
     "blocks = [nb - 1] if (last_block_only and nb > 0) else range(nb)\n        for lb in blocks:\n"
     "            pb = int(block_tables[b, lb])\n            n = min(bs, L - lb * bs)\n            k = e4m3_to_f64",
     "blocks = [0] if (last_block_only and nb > 0) else range(nb)\n        for lb in blocks:\n"
     "            pb = int(block_tables[b, lb])\n            n = min(bs, L - lb * bs)\n            k = e4m3_to_f64"),
    ("fp8 meta: code of the magnitude", "return e4m3_from_f32(np.asarray(values, dtype=np.float64).astype(np.float32))",
     "return e4m3_from_f32(np.abs(np.asarray(values, dtype=np.float64)).astype(np.float32))"),
    ("fp8 score: kmin used for both bounds", "hi = e4m3_to_f64(key_max[pbs, g])", "hi = e4m3_to_f64(key_min[pbs, g])"),
    ("fp8 score: codes taken as integers", "lo = e4m3_to_f64(key_min[pbs, g])",
     "lo = key_min[pbs, g].astype(np.float64)"),
    ("fp8 topk: bf16 scores on the codes", "lambda b, g: quest_block_scores_fp8(",
     "lambda b, g: quest_block_scores("),
    ("varlen: query rows shifted", "s_ = sc * (q[r0:r1, h] @ k[:, g].T)", "s_ = sc * (q[r0 + 1:r1 + 1, h] @ k[:, g].T)"),
]


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC
    exec(compile(src.replace(old, new), SRC + ":mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_killed(name, old, new):
    orc = _mutant(old, new)
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:
            return          # killed
    pytest.fail(f"mutant survived every pin: {name}")
