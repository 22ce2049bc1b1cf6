"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one: a dropped scale, a wrong KV-head map, an off-by-one causal
mask, a transposed operand, a wrong log base, a wrong block walk, swapped K/V
halves, a linear (not exponential) merge weight, a floor in the split count,
an FP8 decoding with the wrong exponent bias, FP8 rounding toward zero,
swapped K/V dequantisation scales, MLA keys expanded with the value columns,
MLA keys without their rope part, the projection's bf16 rounding left out or
done by truncation, the FP8 latent row's rope part stored without its scale,
and the FP8 latent dequantisation without its scale."""
import numpy as np
import pytest

import oracle.pa_oracle as O
import oracle_pins as P

_attention = O.attention
_gather_kv = O.gather_kv
_cache_write_kv = O.cache_write_kv
_lse_merge = O.lse_merge
_num_kv_splits = O.num_kv_splits
_slot_of = O.slot_of


def _attention_variant(kv_map=None, causal_shift=0, use_keys_as_values=False,
                       log2_lse=False, drop_scale=False, no_max=False):
    def attention(q, keys, vals, scale, num_prior):
        L, Hq, _ = q.shape
        S, Hkv, Dv = vals.shape
        group = Hq // Hkv
        out = np.zeros((L, Hq, Dv))
        lse = np.full((L, Hq), -np.inf)
        if S == 0 or L == 0:
            return out, lse
        vis = np.ones((L, S), bool) if num_prior is None else \
            np.arange(S)[None, :] <= (num_prior + causal_shift + np.arange(L))[:, None]
        V = keys if use_keys_as_values else vals
        for h in range(Hq):
            kvh = kv_map(h, Hq, Hkv) if kv_map else h // group
            z = (1.0 if drop_scale else scale) * (q[:, h] @ keys[:, kvh].T)
            z = np.where(vis, z, -np.inf)
            m = np.zeros(L) if no_max else z.max(axis=1)
            w = np.where(vis, np.exp(z - m[:, None]), 0.0)
            den = w.sum(axis=1)
            out[:, h] = (w @ V[:, kvh, :Dv]) / den[:, None]
            lse[:, h] = (m + np.log(den)) / (np.log(2) if log2_lse else 1.0)
        return out, lse
    return attention


def _gather_wrong_walk(cache, row, seq_len):
    bs = cache.shape[2]
    pos = np.arange(seq_len)
    blocks = np.asarray(row)[pos % len(row)].astype(np.int64)   # wrong block index
    return O.to_f64(cache[blocks, 0, pos % bs]), O.to_f64(cache[blocks, 1, pos % bs])


def _write_swapped(cache, k, v, slots):
    return _cache_write_kv(cache, v, k, slots)


def _merge_linear(outs, lses):
    w = np.where(np.isfinite(lses), lses - np.nanmin(np.where(np.isfinite(lses), lses, np.nan)) + 1, 0)
    tot = w.sum(axis=-1)
    return (w[..., None] * outs).sum(axis=-2) / tot[..., None], np.log(tot)


_fp8_dec = O.fp8_e4m3_to_f64
_f32_to_fp8 = O.f32_to_fp8_e4m3
_dequant = O.dequant_kv_cache


def _fp8_bias8(codes):
    """E4M3 decoded with exponent bias 8 (another FP8 variant's)."""
    return _fp8_dec(codes) / 2.0


def _fp8_truncate(x):
    """Round toward zero instead of to nearest."""
    x = np.asarray(x, np.float32)
    table = _fp8_dec(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x).astype(np.float64), 448.0)
    c = np.clip(np.searchsorted(table, a, side="right") - 1, 0, 0x7E).astype(np.uint8)
    return np.where(np.signbit(x), c | np.uint8(0x80), c).astype(np.uint8)


def _dequant_swapped(cache, k_scale, v_scale):
    return _dequant(cache, v_scale, k_scale)


_mla_expand = O.mla_expand


def _expand_swapped_roles(rows, w, qk_nope):
    """Keys expanded with the value rows' block and vice versa."""
    W = np.asarray(w)
    swapped = np.concatenate([W[:, qk_nope:2 * qk_nope], W[:, :qk_nope], W[:, 2 * qk_nope:]], axis=1)
    return _mla_expand(rows, swapped, qk_nope)


def _expand_no_rope(rows, w, qk_nope):
    keys, vals = _mla_expand(rows, w, qk_nope)
    keys = keys.copy()
    keys[:, :, qk_nope:] = 0.0
    return keys, vals


def _round_bf16_truncate(x):
    """Round toward zero to 8 significant bits instead of to nearest."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.trunc(m * 256.0) / 256.0, e)


_quantize_fp8 = O.quantize_fp8
_cache_write_mla = O.cache_write_mla


def _mla_fp8_unscaled_rope(cache, kv_c, k_pe, slots, scale):
    return _cache_write_mla(cache, _quantize_fp8(kv_c, scale), _quantize_fp8(k_pe, 1.0), slots)


MUTATIONS = {
    "drop_scale": ("attention", _attention_variant(drop_scale=True)),
    "kv_head_modulo": ("attention", _attention_variant(kv_map=lambda h, Hq, Hkv: h % Hkv)),
    "causal_off_by_one": ("attention", _attention_variant(causal_shift=-1)),
    "causal_sees_one_future": ("attention", _attention_variant(causal_shift=1)),
    "keys_as_values": ("attention", _attention_variant(use_keys_as_values=True)),
    "lse_log2": ("attention", _attention_variant(log2_lse=True)),
    "wrong_block_walk": ("gather_kv", _gather_wrong_walk),
    "swapped_kv_halves": ("cache_write_kv", _write_swapped),
    "linear_merge_weight": ("lse_merge", _merge_linear),
    "split_count_floor": ("num_kv_splits", lambda m, c: int(min(max(int(m) // 512, 1), 2 * c))),
    "slot_uses_block_size_one": ("slot_of", lambda row, p, bs: int(row[p // bs]) + p % bs),
    "fp8_exponent_bias_8": ("fp8_e4m3_to_f64", _fp8_bias8),
    "fp8_round_toward_zero": ("f32_to_fp8_e4m3", _fp8_truncate),
    "fp8_swapped_plane_scales": ("dequant_kv_cache", _dequant_swapped),
    "mla_expand_swapped_kv_columns": ("mla_expand", _expand_swapped_roles),
    "mla_expand_drops_rope_key": ("mla_expand", _expand_no_rope),
    "bf16_rounding_identity": ("_round_bf16", lambda x: np.asarray(x, np.float64)),
    "bf16_rounding_truncates": ("_round_bf16", _round_bf16_truncate),
    "fp8_mla_rope_unscaled": ("cache_write_mla_fp8", _mla_fp8_unscaled_rope),
    "fp8_mla_dequant_drops_scale": ("dequant_mla_cache", lambda c, s: _fp8_dec(c)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in P.ALL_PINS:
        pin()
