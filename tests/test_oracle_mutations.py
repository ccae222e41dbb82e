"""Planted mistakes in the CPU oracle must each fail at least one pin.

Each mutant replaces one oracle function (on the CPU, via monkeypatch) with a plausible
bug: a dropped term, a wrong sign or index, a transposed or swapped operand. The pins of
tests/oracle_pins.py are then run against the mutated oracle; the test passes only if
some pin rejects it, which shows the pins constrain every step of the oracle.
"""

import numpy as np
import pytest

import oracle.paged_attention as pa
from tests import oracle_pins

_gather = pa.gather_sequence
_attn = pa.attention_one_query


def m_drop_scale(q, K, V, scale):
    return _attn(q, K, V, 1.0)


def m_softmin(q, K, V, scale):
    s = float(scale) * (K @ q.astype(np.float64))
    w = np.exp(-(s - s.min()))
    return (w @ V) / w.sum()


def m_no_normalise(q, K, V, scale):
    s = float(scale) * (K @ q.astype(np.float64))
    w = np.exp(s - s.max())
    return w @ V


def m_weights_on_keys(q, K, V, scale):
    s = float(scale) * (K @ q.astype(np.float64))
    w = np.exp(s - s.max())
    return (w @ K) / w.sum()


def m_mask_short(pool, row, L, h):
    full = _gather(pool, row, L, h)
    return full[:max(int(L) - 1, 1)]


def m_mask_long(pool, row, L, h):
    nb, _, bs, _ = pool.shape
    rows = []
    for j in range(-(-(int(L) + 1) // bs)):
        rows.append(pool[int(row[j]) % nb, h])
    return np.concatenate(rows)[:int(L) + 1].astype(np.float64)


def m_reverse_blocks(pool, row, L, h):
    nb = pa.blocks_needed(L, pool.shape[2])
    rev = np.array(row, copy=True)
    rev[:nb] = rev[:nb][::-1]
    return _gather(pool, rev, L, h)


def m_head_zero(pool, row, L, h):
    return _gather(pool, row, L, 0)


def m_offset_swapped(pool, row, L, h):
    nb_pool, _, bs, _ = pool.shape
    out = []
    for t in range(int(L)):
        j, off = divmod(t, bs)
        out.append(pool[int(row[j]), h, (bs - 1 - off)])
    return np.array(out, np.float64)


def _decode_with_head_map(head_map):
    def paged_decode(q, k_pool, v_pool, block_table, context_lens, scale):
        B, Hq, d = q.shape
        Hkv = k_pool.shape[1]
        out = np.empty((B, Hq, d))
        for b in range(B):
            for h in range(Hq):
                g = head_map(h, Hq, Hkv)
                K = _gather(k_pool, block_table[b], context_lens[b], g)
                V = _gather(v_pool, block_table[b], context_lens[b], g)
                out[b, h] = _attn(q[b, h], K, V, scale)
        return out
    return paged_decode


def m_wrong_sequence_row(q, k_pool, v_pool, block_table, context_lens, scale):
    B = q.shape[0]
    rolled = np.roll(block_table, 1, axis=0) if B > 1 else block_table
    return pa.__dict__["_orig_paged_decode"](q, k_pool, v_pool, rolled, context_lens, scale)


def m_heads_gqa_modulo(q, k_pool, v_pool, block_table, context_lens, scale, pairs):
    Hkv = k_pool.shape[1]
    out = np.empty((len(pairs), q.shape[2]))
    for i, (b, h) in enumerate(pairs):
        K = _gather(k_pool, block_table[b], context_lens[b], h % Hkv)
        V = _gather(v_pool, block_table[b], context_lens[b], h % Hkv)
        out[i] = _attn(q[b, h], K, V, scale)
    return out


def m_window_off_by_one(q, k_pool, v_pool, block_table, context_lens, scale, window):
    return pa.__dict__["_orig_paged_decode_window"](q, k_pool, v_pool, block_table, context_lens, scale,
                                                    int(window) + 1)


def m_window_start_floor_block(L, W):
    lo = max(0, int(L) - int(W))
    return lo - lo % 4


def m_cache_divmod_swapped(k_pool, v_pool, key, value, slot_mapping):
    k_new, v_new = k_pool.copy(), v_pool.copy()
    nb, _, bs, _ = k_pool.shape
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = int(slot) % bs, int(slot) // bs  # block and offset swapped
        if blk >= nb or off >= bs:
            raise pa.OracleInputError("slot")
        k_new[blk, :, off, :] = key[i]
        v_new[blk, :, off, :] = value[i]
    return k_new, v_new


def m_cache_skips_value(k_pool, v_pool, key, value, slot_mapping):
    k_new, _ = pa.__dict__["_orig_reshape_and_cache"](k_pool, v_pool, key, value, slot_mapping)
    return k_new, v_pool.copy()


def m_copy_only_k(k_pool, v_pool, pairs):
    k_new, _ = pa.__dict__["_orig_copy_blocks"](k_pool, v_pool, pairs)
    return k_new, v_pool.copy()


def m_copy_reversed(k_pool, v_pool, pairs):
    p = np.asarray(pairs).reshape(-1, 2)[:, ::-1]
    return pa.__dict__["_orig_copy_blocks"](k_pool, v_pool, p)


def m_bytes_no_factor2(num_kv_heads, head_dim, dtype_bytes, context_lens, num_layers=1):
    return pa.__dict__["_orig_kv_cache_bytes"](num_kv_heads, head_dim, dtype_bytes, context_lens,
                                                num_layers) // 2


def m_blocks_floor(L, bs):
    return int(L) // int(bs)


def m_layer_pools_kv_swapped(cache, layer):
    return cache[:, 1, int(layer)], cache[:, 0, int(layer)]


def m_layer_pools_layer_zero(cache, layer):
    return cache[:, 0, 0], cache[:, 1, 0]


def m_reblock_identity_table(pool, table, lens, nbs, new_table, nnb):
    ident = np.tile(np.arange(np.shape(new_table)[1], dtype=np.int32), (len(lens), 1))
    return pa.__dict__["_orig_reblock"](pool, table, lens, nbs, ident, nnb)


def m_reblock_shifted(pool, table, lens, nbs, new_table, nnb):
    out = pa.__dict__["_orig_reblock"](pool, table, lens, nbs, new_table, nnb)
    return np.roll(out, 1, axis=2)


def m_compact_no_relabel(k_pool, v_pool, table, pairs):
    k2, v2, _ = pa.__dict__["_orig_compact_blocks"](k_pool, v_pool, table, pairs)
    return k2, v2, np.array(table, copy=True)


def m_compact_copy_reversed(k_pool, v_pool, table, pairs):
    p = np.asarray(pairs).reshape(-1, 2)[:, ::-1]
    k2, v2 = pa.__dict__["_orig_copy_blocks"](k_pool, v_pool, p)
    _, _, t2 = pa.__dict__["_orig_compact_blocks"](k_pool, v_pool, table, pairs)
    return k2, v2, t2


def _multi_with_position(shift):
    def paged_attention_multi(q, k_pool, v_pool, block_table, context_lens, query_start, scale):
        T, Hq, d = q.shape
        Hkv = k_pool.shape[1]
        G = Hq // Hkv
        qs = np.asarray(query_start)
        out = np.full((T, Hq, d), np.nan)
        for b, L in enumerate(context_lens):
            n = int(qs[b + 1] - qs[b])
            for g in range(Hkv):
                K = _gather(k_pool, block_table[b], L, g)
                V = _gather(v_pool, block_table[b], L, g)
                for i in range(n):
                    p = min(max(int(L) - n + i + shift(i, n, int(L)), 0), int(L) - 1)
                    for h in range(g * G, (g + 1) * G):
                        out[qs[b] + i, h] = _attn(q[qs[b] + i, h], K[:p + 1], V[:p + 1], scale)
        return out
    return paged_attention_multi


MUTANTS = {
    "drop_scale": ("attention_one_query", m_drop_scale),
    "softmin": ("attention_one_query", m_softmin),
    "no_normalise": ("attention_one_query", m_no_normalise),
    "weights_on_keys": ("attention_one_query", m_weights_on_keys),
    "mask_short": ("gather_sequence", m_mask_short),
    "mask_long": ("gather_sequence", m_mask_long),
    "reverse_blocks": ("gather_sequence", m_reverse_blocks),
    "head_zero": ("gather_sequence", m_head_zero),
    "offset_swapped": ("gather_sequence", m_offset_swapped),
    "gqa_modulo": ("paged_decode", _decode_with_head_map(lambda h, Hq, Hkv: h % Hkv)),
    "gqa_identity": ("paged_decode", _decode_with_head_map(lambda h, Hq, Hkv: min(h, Hkv - 1))),
    "wrong_sequence_row": ("paged_decode", m_wrong_sequence_row),
    "heads_gqa_modulo": ("paged_decode_heads", m_heads_gqa_modulo),
    "window_off_by_one": ("paged_decode_window", m_window_off_by_one),
    "window_start_block_floor": ("window_start", m_window_start_floor_block),
    "cache_divmod_swapped": ("reshape_and_cache", m_cache_divmod_swapped),
    "cache_skips_value": ("reshape_and_cache", m_cache_skips_value),
    "copy_only_k": ("copy_blocks", m_copy_only_k),
    "copy_reversed": ("copy_blocks", m_copy_reversed),
    "bytes_no_factor2": ("kv_cache_bytes", m_bytes_no_factor2),
    "blocks_floor": ("blocks_needed", m_blocks_floor),
    "layer_pools_kv_swapped": ("layer_pools", m_layer_pools_kv_swapped),
    "layer_pools_layer_zero": ("layer_pools", m_layer_pools_layer_zero),
    "reblock_identity_table": ("reblock", m_reblock_identity_table),
    "reblock_shifted": ("reblock", m_reblock_shifted),
    "compact_no_relabel": ("compact_blocks", m_compact_no_relabel),
    "compact_copy_reversed": ("compact_blocks", m_compact_copy_reversed),
    "multi_no_causal_mask": ("paged_attention_multi", _multi_with_position(lambda i, n, L: n - 1 - i)),
    "multi_mask_one_short": ("paged_attention_multi", _multi_with_position(lambda i, n, L: -1)),
    "multi_forgets_history": ("paged_attention_multi", _multi_with_position(lambda i, n, L: n - L)),
}


def _run_pins(pins, module, name):
    """Run every pin against the mutated oracle; returns the pins that rejected it.

    A kill is a value check that fails (AssertionError) or the oracle's own input check
    raising where the pages call for none (OracleInputError). Any other exception is a crash
    of the mutant, not evidence that a pin noticed wrong numbers: it is reported and does not
    count, so the mutant must still fail some pin's value check."""
    failed = []
    for pin in pins:
        try:
            pin(module)
        except (AssertionError, pa.OracleInputError) as e:
            failed.append((pin.__name__, type(e).__name__))
        except Exception as e:  # noqa: BLE001
            print(f"mutant {name}: pin {pin.__name__} crashed ({type(e).__name__}: {e}); not counted as a kill")
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    for orig in ("paged_decode", "reshape_and_cache", "copy_blocks", "kv_cache_bytes",
                 "paged_decode_window", "reblock", "compact_blocks"):
        monkeypatch.setitem(pa.__dict__, "_orig_" + orig, getattr(pa, orig))
    monkeypatch.setattr(pa, attr, fn)
    failed = _run_pins(oracle_pins.ALL_PINS, pa, name)
    assert failed, f"mutant {name} passed every pin"


# ---- planted mistakes in the 8-bit float cache oracle ---------------------------------------

import oracle.fp8_cache as o8  # noqa: E402

_value = o8.e4m3_value
_encode = o8.e4m3_encode
_quantize = o8.quantize_rows
_dequantize = o8.dequantize
_append8 = o8.reshape_and_cache_fp8
_copy8 = o8.copy_blocks_fp8


def m8_bias_8(codes):
    # the other common 8-bit float flavour: exponent bias 8
    return _value(codes) / 2.0


def m8_no_subnormals(codes):
    c = np.asarray(codes, np.int64)
    v = _value(codes)
    return np.where(((c >> 3) & 0xF) == 0, 0.0 * v, v)


def m8_ties_away(x):
    x = np.asarray(x, np.float64)
    mags = _value(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(x)
    hi = np.minimum(np.searchsorted(mags, a), len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    code = np.where(mags[hi] - a <= a - mags[lo], hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def m8_truncate(x):
    x = np.asarray(x, np.float64)
    mags = _value(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(x)
    code = np.searchsorted(mags, a, side="right") - 1
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def m8_scale_127(x):
    # an int8-style scale: s = max|x| / 127, so codes never reach the top of the range
    x = np.asarray(x, np.float32)
    s = (np.max(np.abs(x), axis=-1) / np.float32(127.0)).astype(np.float32)
    quot = (x / np.where(s == 0, np.float32(1), s)[..., None]).astype(np.float32)
    codes = np.where((s == 0)[..., None], np.uint8(0), o8.e4m3_encode(quot)).astype(np.uint8)
    return codes, s


def m8_dequant_no_scale(codes, scales):
    return _value(codes)


def m8_dequant_scale_shifted(codes, scales):
    return _value(codes) * np.roll(np.asarray(scales, np.float64), 1, axis=-1)[..., None]


def m8_append_scale_misplaced(kc, vc, ks, vs, key, value, slots):
    k2, v2, ks2, vs2 = _append8(kc, vc, ks, vs, key, value, slots)
    return k2, v2, np.roll(ks2, 1, axis=-1), vs2


def m8_append_v_from_k(kc, vc, ks, vs, key, value, slots):
    return _append8(kc, vc, ks, vs, key, key, slots)


def m8_copy_without_scales(kc, vc, ks, vs, pairs):
    k2, v2, _, _ = _copy8(kc, vc, ks, vs, pairs)
    return k2, v2, ks.copy(), vs.copy()


FP8_MUTANTS = {
    "bias_8": ("e4m3_value", m8_bias_8),
    "no_subnormals": ("e4m3_value", m8_no_subnormals),
    "ties_away": ("e4m3_encode", m8_ties_away),
    "truncate": ("e4m3_encode", m8_truncate),
    "scale_127": ("quantize_rows", m8_scale_127),
    "dequant_no_scale": ("dequantize", m8_dequant_no_scale),
    "dequant_scale_shifted": ("dequantize", m8_dequant_scale_shifted),
    "append_scale_misplaced": ("reshape_and_cache_fp8", m8_append_scale_misplaced),
    "append_v_from_k": ("reshape_and_cache_fp8", m8_append_v_from_k),
    "copy_without_scales": ("copy_blocks_fp8", m8_copy_without_scales),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(o8, attr, fn)
    failed = _run_pins(oracle_pins.FP8_PINS, o8, name)
    assert failed, f"mutant {name} passed every pin"
