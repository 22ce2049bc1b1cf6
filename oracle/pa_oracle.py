"""Float64 CPU oracle for paged KV attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the CPU-baseline leg of ``bench.py`` may import
this module.  The HIP library and its Python binding never import it, and it
imports nothing from them.  It shares no code, tables or helpers with the GPU
path: the only thing both sides see is the seeded input generator, which holds
none of the attention arithmetic.

What is computed, and where the pages define it
-----------------------------------------------
* Cache write.  "Attention Backends" (infra.riteshsonawane.com), section
  "What paged attention requires of a kernel", step 1: the T new keys and
  values are stored in the cache at ``slot_mapping``.  A slot is the flat
  index ``physical_block * block_size + offset``; the "Code" section of the
  same page builds it as ``blockTable[pos/blockSize]*blockSize +
  pos%blockSize``.  The GQA cache layout ``[num_blocks, 2, block_size,
  num_kv_heads, head_size]`` and the MLA layout ``[num_blocks, block_size,
  head_size]`` are from "AttentionBackend：注意力后端抽象层", section 设计动机.
* Gather through the block table.  Same "Attention Backends" page, step 2 and
  the ``pagedAttend`` function of its "Code" section: position p of a request
  lives at block ``block_table[p // block_size]``, offset ``p % block_size``;
  only the first ``seq_len`` positions take part.
* Attention.  "第 1 章 注意力后端", §2.1 (the formula
  O = softmax(Q K^T / sqrt(d_h) + M) V, M the causal mask).  The oracle is that
  definition written out in float64: scores, row max, exponentials, sum,
  weighted sum of V.  The log-sum-exp of the scaled scores (natural log) is
  returned beside the output ("AttentionBackend：注意力后端抽象层", 设计动机 and
  边界与失败: lse must be in base e for cross-shard merges).
* GQA head sharing.  "第 1 章 注意力后端", §3.2: several query heads share one
  KV head.  Reading: query head h uses KV head ``h // (Hq // Hkv)``.
* Split-KV merge.  "第 1 章 注意力后端", §3.1 (split-KV, partial outputs merged
  with their softmax normalisers) and §4.1 Figure 5c (a block's earlier
  contribution is re-weighted when a new block joins).  The merge is the exact
  identity  out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M),
  lse = M + ln sum_s exp(lse_s - M), M = max_s lse_s.
* MLA.  "Triton 與 MLA：可移植注意力與潛空間注意力", sections 設計動機 and 資料流:
  the cache row is ``[kv_c (kv_lora_rank) | k_pe (rope)]``, read as a single
  MQA key head; the query is ``cat(q_nope, q_pe)``; V is the first
  kv_lora_rank columns of the same row; the output has kv_lora_rank columns.
* Split count.  Same Triton/MLA page, section 關鍵檔案 (``_compute_num_kv_splits``):
  ``max_seq_len / 512`` splits, capped at twice the compute-unit count.
* FP8 cache.  Same Triton/MLA page, 資料流 (the layer's k_scale / v_scale go
  to the kernel; v_scale = k_scale for the latent cache) and 邊界與失敗 (the
  query stays bf16; the kernel dequantises).  Format and rounding are a
  reading (OCP E4M3, round to nearest even, saturating), stated at the
  functions.

Readings where the pages leave a step open (each is also listed in the design doc):
* ``seq_len`` includes this step's new tokens (the write happens first), and
  a request's new tokens are its last ``L_r`` positions.
* Causal alignment is bottom-right: query i of a chunk of L_r new tokens over
  S_r keys sees keys j <= (S_r - L_r) + i.
* A negative slot means "do not write".
* A row that sees no key gets out = 0 and lse = -inf; an empty split has
  lse = -inf and weight 0 in the merge.
* The split count rounds up: ceil(max_seq_len / 512), at least 1.

Storage conventions: bf16 tensors are passed as ``numpy.uint16`` arrays of raw
bf16 bits; fp32 tensors as ``numpy.float32``.  Every arithmetic result is
float64 and is not rounded to the storage type.
"""

from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------
# storage decoding
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of raw bf16 bits: the bits are the top half of an IEEE fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Decode a stored tensor (uint16 = bf16 bits, float32, float64) to float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype}")


# --------------------------------------------------------------------------
# step 1: the cache write
# --------------------------------------------------------------------------

def cache_write_kv(cache: np.ndarray, k: np.ndarray, v: np.ndarray,
                   slot_mapping: np.ndarray) -> np.ndarray:
    """Return a copy of a GQA cache after storing new keys/values at their slots.

    cache: [num_blocks, 2, block_size, num_kv_heads, head_dim] (index 0 = K,
    index 1 = V); k, v: [T, num_kv_heads, head_dim] in the cache's storage
    dtype; slot_mapping: [T] int64.  ("Attention Backends", "What paged
    attention requires of a kernel", step 1.)  The copy is byte for byte.
    """
    out = cache.copy()
    block_size = cache.shape[2]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        out[blk, 0, off] = k[t]
        out[blk, 1, off] = v[t]
    return out


def cache_write_mla(cache: np.ndarray, kv_c: np.ndarray, k_pe: np.ndarray,
                    slot_mapping: np.ndarray) -> np.ndarray:
    """Return a copy of an MLA latent cache after storing new rows.

    cache: [num_blocks, block_size, kv_lora_rank + rope_dim]; kv_c:
    [T, kv_lora_rank]; k_pe: [T, rope_dim].  The stored row is kv_c followed
    by k_pe ("Triton 與 MLA", 資料流).
    """
    out = cache.copy()
    block_size = cache.shape[1]
    rank = kv_c.shape[1]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        out[blk, off, :rank] = kv_c[t]
        out[blk, off, rank:] = k_pe[t]
    return out


# --------------------------------------------------------------------------
# step 2: gather a request's first seq_len positions through its block table
# --------------------------------------------------------------------------

def gather_kv(cache: np.ndarray, block_table_row: np.ndarray, seq_len: int):
    """Keys and values of positions 0..seq_len-1 of one request, as float64.

    Position p is at block ``block_table_row[p // block_size]``, offset
    ``p % block_size`` ("Attention Backends", ``pagedAttend`` in "Code").
    Returns K, V of shape [seq_len, num_kv_heads, head_dim].
    """
    block_size = cache.shape[2]
    pos = np.arange(seq_len)
    blocks = np.asarray(block_table_row)[pos // block_size].astype(np.int64)
    offs = pos % block_size
    keys = cache[blocks, 0, offs]
    vals = cache[blocks, 1, offs]
    return to_f64(keys), to_f64(vals)


def gather_mla(cache: np.ndarray, block_table_row: np.ndarray, seq_len: int):
    """Latent rows of positions 0..seq_len-1 of one request: [seq_len, row] f64."""
    block_size = cache.shape[1]
    pos = np.arange(seq_len)
    blocks = np.asarray(block_table_row)[pos // block_size].astype(np.int64)
    return to_f64(cache[blocks, pos % block_size])


# --------------------------------------------------------------------------
# attention over gathered keys (the formula of 第 1 章 §2.1)
# --------------------------------------------------------------------------

def attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float,
              num_prior: int | None):
    """softmax(scale * Q K^T + M) V and its natural-log normaliser.

    q: [L, Hq, Dk]; keys: [S, Hkv, Dk]; vals: [S, Hkv, Dv] (all float64).
    Query head h reads KV head h // (Hq // Hkv).
    num_prior = None: no mask (every query sees all S keys).  Otherwise query i
    sees keys j <= num_prior + i (causal, bottom-right aligned).
    Returns out [L, Hq, Dv] and lse [L, Hq]; a row that sees no key gets
    out = 0 and lse = -inf.
    """
    L, Hq, _ = q.shape
    S, Hkv, Dv = vals.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    out = np.zeros((L, Hq, Dv), dtype=np.float64)
    lse = np.full((L, Hq), NEG_INF, dtype=np.float64)
    if S == 0 or L == 0:
        return out, lse
    if num_prior is None:
        visible = np.ones((L, S), dtype=bool)
    else:
        visible = np.arange(S)[None, :] <= (num_prior + np.arange(L))[:, None]
    for h in range(Hq):
        kvh = h // group
        z = scale * (q[:, h, :] @ keys[:, kvh, :].T)          # [L, S]
        z = np.where(visible, z, NEG_INF)
        m = z.max(axis=1)                                    # row max
        ok = np.isfinite(m)
        w = np.where(visible, np.exp(z - np.where(ok, m, 0.0)[:, None]), 0.0)
        denom = w.sum(axis=1)
        num = w @ vals[:, kvh, :]                             # [L, Dv]
        out[ok, h, :] = num[ok] / denom[ok, None]
        lse[ok, h] = m[ok] + np.log(denom[ok])
    return out, lse


# --------------------------------------------------------------------------
# whole operations over a batch
# --------------------------------------------------------------------------

def paged_attention(q, cache, block_table, query_start_loc, seq_lens, scale,
                    causal=True, requests=None):
    """Varlen paged attention over a GQA cache (already written).

    q: [T, Hq, D] storage dtype; cache [nb, 2, bs, Hkv, D]; block_table
    [N, max_blocks] int32; query_start_loc [N+1]; seq_lens [N].
    Request r owns query rows query_start_loc[r] .. query_start_loc[r+1]-1,
    which are its last L_r positions; causal attention is bottom-right
    aligned.  Decode is the case L_r = 1 for every request.
    ``requests``: optional subset of request indices to evaluate (the rest of
    the output is left as NaN).
    Returns out [T, Hq, D] and lse [T, Hq] (float64).
    """
    T, Hq, _ = q.shape
    Dv = cache.shape[-1]
    out = np.full((T, Hq, Dv), np.nan)
    lse = np.full((T, Hq), np.nan)
    n = len(seq_lens)
    for r in (range(n) if requests is None else requests):
        a, b = int(query_start_loc[r]), int(query_start_loc[r + 1])
        S = int(seq_lens[r])
        L = b - a
        keys, vals = gather_kv(cache, block_table[r], S)
        o, l = attention(to_f64(q[a:b]), keys, vals, scale,
                         (S - L) if causal else None)
        out[a:b], lse[a:b] = o, l
    return out, lse


def paged_decode(q, cache, block_table, seq_lens, scale, requests=None):
    """Decode: one query per request.  q [B, Hq, D] -> out [B, Hq, D], lse [B, Hq]."""
    qsl = np.arange(len(seq_lens) + 1)
    return paged_attention(q, cache, block_table, qsl, seq_lens, scale,
                           causal=True, requests=requests)


def mla_decode(q_nope, q_pe, cache, block_table, seq_lens, scale, requests=None):
    """MLA decode over the latent cache, read as one shared key head.

    q_nope [B, H, R], q_pe [B, H, P]; cache [nb, bs, R+P].  K is the full
    R+P row, V its first R columns ("Triton 與 MLA", 資料流).
    Returns out [B, H, R] and lse [B, H] (float64).
    """
    B, H, R = q_nope.shape
    out = np.full((B, H, R), np.nan)
    lse = np.full((B, H), np.nan)
    for r in (range(B) if requests is None else requests):
        S = int(seq_lens[r])
        rows = gather_mla(cache, block_table[r], S)          # [S, R+P]
        q = np.concatenate([to_f64(q_nope[r]), to_f64(q_pe[r])], axis=-1)
        o, l = attention(q[None], rows[:, None, :], rows[:, None, :R], scale, S - 1)
        out[r], lse[r] = o[0], l[0]
    return out, lse


# --------------------------------------------------------------------------
# split-KV partials and their merge (第 1 章 §3.1, §4.1 Figure 5c)
# --------------------------------------------------------------------------

def partial_attention(q, keys, vals, scale, lo, hi, num_prior):
    """Attention restricted to key positions lo..hi-1 (a KV split).

    Positions keep their absolute index for the causal mask.  Returns the
    split's own normalised output and its lse (lse = -inf if it sees nothing).
    """
    L = q.shape[0]
    S = keys.shape[0]
    if num_prior is None:
        vis_hi = np.full(L, S)
    else:
        vis_hi = num_prior + np.arange(L) + 1
    Hq = q.shape[1]
    Dv = vals.shape[2]
    out = np.zeros((L, Hq, Dv))
    lse = np.full((L, Hq), NEG_INF)
    for i in range(L):
        top = min(hi, int(vis_hi[i]))
        if top <= lo:
            continue
        o, l = attention(q[i:i + 1], keys[lo:top], vals[lo:top], scale, None)
        out[i], lse[i] = o[0], l[0]
    return out, lse


def lse_merge(outs: np.ndarray, lses: np.ndarray):
    """Merge split partials along axis -2 of ``outs`` / axis -1 of ``lses``.

    outs: [..., S, Dv]; lses: [..., S].  Exact identity of the split softmax:
    weights exp(lse_s - M), M the largest lse; -inf splits weigh 0; if every
    split is -inf the result is out = 0, lse = -inf.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=-1)
    ok = np.isfinite(M)
    Ms = np.where(ok, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms[..., None]), 0.0)
    tot = w.sum(axis=-1)
    safe = np.where(ok, tot, 1.0)
    out = np.where(ok[..., None], (w[..., None] * outs).sum(axis=-2) / safe[..., None], 0.0)
    lse = np.where(ok, Ms + np.log(safe), NEG_INF)
    return out, lse


def lse_merge_packed(part: np.ndarray):
    """Merge the packed workspace format [..., S, Dv+1] (lse at index Dv)."""
    part = np.asarray(part, dtype=np.float64)
    return lse_merge(part[..., :-1], part[..., -1])


# --------------------------------------------------------------------------
# host integer helpers
# --------------------------------------------------------------------------

def num_kv_splits(max_seq_len: int, num_cus: int) -> int:
    """ceil(max_seq_len / 512), at least 1, at most 2 * num_cus
    ("Triton 與 MLA", 關鍵檔案: ``_compute_num_kv_splits``)."""
    n = -(-int(max_seq_len) // 512)
    return int(min(max(n, 1), 2 * int(num_cus)))


def slot_of(block_table_row, pos: int, block_size: int) -> int:
    """Flat slot of logical position ``pos`` ("Attention Backends", "Code")."""
    return int(block_table_row[pos // block_size]) * block_size + pos % block_size


# --------------------------------------------------------------------------
# MLA prefill: the multi-head form over expanded keys and values
# --------------------------------------------------------------------------
# "Triton 與 MLA" (設計動機, 關鍵檔案): the MLA layer holds kv_b_proj,
# qk_nope_head_dim, qk_rope_head_dim and kv_lora_rank, and its backend has two
# entry points, forward_mqa (decode, over the latent rows) and forward_mha;
# "Attention Backends" ("Latent attention is a different cache"): prefill and
# decode use different formulations of the same mathematics.  Reading of the
# multi-head form: per head h, the key of position j is
# [W_k[h] kv_c_j | k_pe_j] (qk_nope + rope wide) and its value W_v[h] kv_c_j
# (v_head wide), with kv_b_proj's weight stored as a linear layer stores it,
# [H * (qk_nope + v), kv_lora_rank] = [H, qk_nope + v, kv_lora_rank] (W_k the
# first qk_nope output rows of each head, W_v the rest); expanded keys
# and values are the projection's output, a bf16 tensor (each element the
# exact product rounded to nearest even); the query is [q_nope | q_pe] per
# head; causal attention as in ``paged_attention``.

def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 value of float64 numbers (exact arithmetic on the
    float32 rounding: a float64 -> float32 -> bf16 double rounding is avoided
    by rounding the float64 value directly)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m 2^e, 0.5 <= |m| < 1
    q = np.round(m * 256.0) / 256.0       # 8 significant bits, ties to even
    return np.ldexp(q, e)


def mla_expand(latent_rows: np.ndarray, w_kv_b: np.ndarray, qk_nope: int):
    """Keys and values of the multi-head form from latent rows [S, R + P]:
    keys [S, H, qk_nope + P] and values [S, H, v] (bf16 values as float64).
    w_kv_b: [H, qk_nope + v, R]."""
    R = w_kv_b.shape[2]
    kv_c, k_pe = latent_rows[:, :R], latent_rows[:, R:]
    W = to_f64(w_kv_b)                                       # [H, qk_nope + v, R]
    kv = _round_bf16(np.einsum("sr,hcr->shc", kv_c, W))      # [S, H, qk_nope + v]
    S, H, _ = kv.shape
    keys = np.concatenate([kv[:, :, :qk_nope], np.broadcast_to(k_pe[:, None, :], (S, H, k_pe.shape[1]))],
                          axis=-1)
    return keys, kv[:, :, qk_nope:]


def mla_prefill(q, cache, w_kv_b, block_table, query_start_loc, seq_lens, scale,
                qk_nope: int = 128, causal: bool = True, requests=None):
    """MLA prefill in the multi-head form over the latent cache (already
    written).  q [T, H, qk_nope + P]; cache [nb, bs, R + P]; w_kv_b
    [H, qk_nope + v, R].  Returns out [T, H, v] and lse [T, H] (float64)."""
    T, H, _ = q.shape
    v_dim = w_kv_b.shape[1] - qk_nope
    out = np.full((T, H, v_dim), np.nan)
    lse = np.full((T, H), np.nan)
    for r in (range(len(seq_lens)) if requests is None else requests):
        a, b = int(query_start_loc[r]), int(query_start_loc[r + 1])
        S = int(seq_lens[r])
        keys, vals = mla_expand(gather_mla(cache, block_table[r], S), w_kv_b, qk_nope)
        o, l = attention(to_f64(q[a:b]), keys, vals, scale, (S - (b - a)) if causal else None)
        out[a:b], lse[a:b] = o, l
    return out, lse


# --------------------------------------------------------------------------
# FP8 KV cache with per-tensor scales
# --------------------------------------------------------------------------
# The pages name an FP8 cache read with per-layer k_scale / v_scale while the
# query stays bf16 ("Triton 與 MLA", 資料流 passes k_scale and v_scale to the
# kernel, v_scale = k_scale for the latent cache; 邊界與失敗: with an FP8 cache
# the kernel dequantises and the query is not quantised).  They do not fix
# the format or the rounding.  Reading: OCP FP8 E4M3 -- 1 sign bit, 4 exponent
# bits with bias 7, 3 mantissa bits, subnormals m * 2^-9, no infinities,
# S.1111.111 is NaN, largest finite 448.  A stored code is E4M3(x / scale)
# with the quotient formed in fp32 (x is a bf16 value, exact in fp32) and
# rounded to the nearest E4M3 value, ties to the even code, saturating at
# +-448; the value read back is E4M3(code) * scale.

def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of E4M3 codes (uint8) by the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    val = np.where(e == 0, sub, normal)
    val = np.where(sign == 1, -val, val)
    return np.where((e == 15) & (m == 7), np.nan, val)


_E4M3_POS = fp8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))   # codes 0..126, increasing


def f32_to_fp8_e4m3(x) -> np.ndarray:
    """E4M3 code of float32 values: nearest value, ties to the even code,
    magnitudes above 448 saturated to 448, NaN to 0x7F; the sign bit is
    kept (so -0 and negatives that round to zero give 0x80)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x).astype(np.float64), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize_fp8(x_bits_bf16, scale: float) -> np.ndarray:
    """Codes of bf16 values divided by ``scale`` (the quotient in fp32)."""
    q = (bf16_bits_to_f64(x_bits_bf16).astype(np.float32) / np.float32(scale)).astype(np.float32)
    return f32_to_fp8_e4m3(q)


def cache_write_kv_fp8(cache: np.ndarray, k: np.ndarray, v: np.ndarray,
                       slot_mapping: np.ndarray, k_scale: float, v_scale: float) -> np.ndarray:
    """The GQA cache write of an FP8 cache (uint8 codes, same layout): new bf16
    keys and values quantised with k_scale / v_scale, then stored at their
    slots as in ``cache_write_kv``."""
    return cache_write_kv(cache, quantize_fp8(k, k_scale), quantize_fp8(v, v_scale),
                          slot_mapping)


def cache_write_mla_fp8(cache: np.ndarray, kv_c: np.ndarray, k_pe: np.ndarray,
                        slot_mapping: np.ndarray, scale: float) -> np.ndarray:
    """The MLA latent write of an FP8 cache: the whole row uses one scale
    ("Triton 與 MLA", 資料流: v_scale = k_scale for the latent cache)."""
    return cache_write_mla(cache, quantize_fp8(kv_c, scale), quantize_fp8(k_pe, scale),
                           slot_mapping)


def dequant_kv_cache(cache: np.ndarray, k_scale: float, v_scale: float) -> np.ndarray:
    """Values an FP8 GQA cache holds: plane 0 times k_scale, plane 1 times
    v_scale, as float64 (for ``paged_attention`` / ``paged_decode``)."""
    out = fp8_e4m3_to_f64(cache)
    out[:, 0] *= float(k_scale)
    out[:, 1] *= float(v_scale)
    return out


def dequant_mla_cache(cache: np.ndarray, scale: float) -> np.ndarray:
    """Values an FP8 latent cache holds, as float64 (for ``mla_decode``)."""
    return fp8_e4m3_to_f64(cache) * float(scale)


__all__ = [
    "bf16_bits_to_f64", "to_f64", "cache_write_kv", "cache_write_mla",
    "gather_kv", "gather_mla", "attention", "paged_attention", "paged_decode",
    "mla_decode", "partial_attention", "lse_merge", "lse_merge_packed",
    "num_kv_splits", "slot_of", "fp8_e4m3_to_f64", "f32_to_fp8_e4m3", "quantize_fp8",
    "cache_write_kv_fp8", "cache_write_mla_fp8", "dequant_kv_cache", "dequant_mla_cache",
    "mla_expand", "mla_prefill",
]
