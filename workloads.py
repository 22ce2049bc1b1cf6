"""Seeded synthetic inputs for the paged-attention workloads.

Shared by the tests, ``bench.py`` and the smoke check: the HIP path and the
CPU oracle both consume exactly these arrays.  This module holds no attention
arithmetic -- only random draws, block allocation, slot bookkeeping (what a
serving engine's cache manager hands to the kernel) and the byte/flop counts
used to price a measurement.

Recipe (all workloads):
* ``numpy.random.default_rng(seed)`` (PCG64).  Named workloads use seed
  1000 + workload number.
* Values are N(0, 1).  fp32 tensors are float32 draws of
  ``standard_normal``.  bf16 tensors (stored as raw ``uint16`` bits) are drawn
  by inverse CDF: a uniform 16-bit integer u selects the N(0, 1) quantile at
  probability (u + 0.5) / 65536, rounded to bf16 nearest-even.  That is N(0, 1)
  at bf16 resolution with tails cut at about 4.3 sigma, and it draws a 2 GiB
  pool an order of magnitude faster than rounding float32 normals.
* The pool holds exactly the blocks the batch needs plus one extra "poison"
  block; block ids are a random permutation, dealt to requests in order.
  Prior-context slots hold N(0, 1) values; every other slot (the slots the
  step's new tokens will be written to, page tails past seq_len, the poison
  block, unassigned blocks) holds NaN, so a kernel that reads anything it
  should not returns NaN.  Block-table padding points at the poison block.
* A request's new tokens are its last L_r positions; seq_len includes them.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"
FP8 = "fp8_e4m3"   # an FP8 cache: q, new k/v and out stay bf16

NAN_BF16 = np.uint16(0x7FC0)
NAN_FP8 = np.uint8(0x7F)      # E4M3 NaN
FP8_MAX_CODE = 0x50           # codes 0x00..0x50: magnitudes 0 .. 8 (exponent field <= 10)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = NAN_BF16
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


_BF16_NORMAL_TABLE = None


def _bf16_normal_table() -> np.ndarray:
    global _BF16_NORMAL_TABLE
    if _BF16_NORMAL_TABLE is None:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _BF16_NORMAL_TABLE = f32_to_bf16_bits(ndtri(p).astype(np.float32))
    return _BF16_NORMAL_TABLE


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    if dtype == BF16:
        u = rng.integers(0, 65536, size=shape, dtype=np.uint16)
        return _bf16_normal_table()[u]
    return rng.standard_normal(size=shape, dtype=np.float32)


def _nan(dtype: str):
    if dtype == FP8:
        return NAN_FP8
    return NAN_BF16 if dtype == BF16 else np.float32(np.nan)


def _fp8_codes(rng, n):
    """Uniformly drawn finite E4M3 codes of magnitude at most 8, either sign."""
    u = rng.integers(0, 2 * (FP8_MAX_CODE + 1), size=n, dtype=np.int32)
    mag = u % (FP8_MAX_CODE + 1)
    return (mag | ((u > FP8_MAX_CODE).astype(np.int32) << 7)).astype(np.uint8)


def _fill_pool(rng, pool_shape, dtype, chunk_blocks=512):
    """Pool of N(0,1) values, filled block-chunk by block-chunk so that a
    2 GiB pool never needs a multi-GiB temporary."""
    nb = pool_shape[0]
    store = {BF16: np.uint16, F32: np.float32, FP8: np.uint8}[dtype]
    pool = np.empty(pool_shape, dtype=store)
    per_block = int(np.prod(pool_shape[1:]))
    flat = pool.reshape(nb, per_block)
    table = _bf16_normal_table() if dtype == BF16 else None
    for b0 in range(0, nb, chunk_blocks):
        b1 = min(nb, b0 + chunk_blocks)
        if dtype == BF16:
            u = rng.integers(0, 65536, size=(b1 - b0) * per_block, dtype=np.uint16)
            flat[b0:b1] = table[u].reshape(b1 - b0, per_block)
        elif dtype == FP8:
            flat[b0:b1] = _fp8_codes(rng, (b1 - b0) * per_block).reshape(b1 - b0, per_block)
        else:
            flat[b0:b1] = rng.standard_normal(size=(b1 - b0, per_block), dtype=np.float32)
    return pool


@dataclass
class GqaBatch:
    """Inputs of one paged GQA call (decode is the case q_len = 1 everywhere).

    Shapes: q [T, Hq, D]; k_new, v_new [T, Hkv, D]; cache [nb, 2, bs, Hkv, D]
    (index 0 = K, 1 = V), holding the prior context only; block_table
    [N, max_blocks] int32; slot_mapping [T] int64; query_start_loc [N+1]
    int32; seq_lens [N] int32.
    """
    name: str
    dtype: str
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    cache: np.ndarray
    block_table: np.ndarray
    slot_mapping: np.ndarray
    query_start_loc: np.ndarray
    seq_lens: np.ndarray
    scale: float
    block_size: int
    poison_block: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self): return len(self.seq_lens)
    @property
    def num_tokens(self): return self.q.shape[0]
    @property
    def num_q_heads(self): return self.q.shape[1]
    @property
    def num_kv_heads(self): return self.cache.shape[3]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def num_blocks(self): return self.cache.shape[0]
    @property
    def q_lens(self): return np.diff(self.query_start_loc)
    @property
    def max_seq_len(self): return int(self.seq_lens.max()) if len(self.seq_lens) else 0
    @property
    def max_query_len(self): return int(self.q_lens.max()) if len(self.seq_lens) else 0
    @property
    def elem_bytes(self): return 4 if self.dtype == F32 else 2      # q / out / new rows
    @property
    def cache_elem_bytes(self): return {BF16: 2, F32: 4, FP8: 1}[self.dtype]
    @property
    def k_scale(self): return self.meta.get("k_scale", 1.0)
    @property
    def v_scale(self): return self.meta.get("v_scale", 1.0)


@dataclass
class MlaBatch:
    """Inputs of one MLA decode call.

    q_nope [B, H, R]; q_pe [B, H, P]; kv_c_new [B, R]; k_pe_new [B, P];
    cache [nb, bs, R+P]; block_table [B, max_blocks]; slot_mapping [B];
    seq_lens [B].  bf16 throughout.
    """
    name: str
    q_nope: np.ndarray
    q_pe: np.ndarray
    kv_c_new: np.ndarray
    k_pe_new: np.ndarray
    cache: np.ndarray
    block_table: np.ndarray
    slot_mapping: np.ndarray
    seq_lens: np.ndarray
    scale: float
    block_size: int
    poison_block: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self): return len(self.seq_lens)
    @property
    def num_heads(self): return self.q_nope.shape[1]
    @property
    def kv_lora_rank(self): return self.q_nope.shape[2]
    @property
    def rope_dim(self): return self.q_pe.shape[2]
    @property
    def num_blocks(self): return self.cache.shape[0]
    @property
    def max_seq_len(self): return int(self.seq_lens.max()) if len(self.seq_lens) else 0
    @property
    def fp8(self): return self.meta.get("cache_dtype") == FP8
    @property
    def cache_elem_bytes(self): return 1 if self.fp8 else 2
    @property
    def kv_scale(self): return self.meta.get("kv_scale", 1.0)


def _allocate_tables(rng, seq_lens, block_size, num_blocks=None, sample_distinct=False):
    """Deal physical blocks to requests; returns (block_table, poison, nb, owned).

    Default: pool of exactly sum(ceil(S_r/bs)) + 1 blocks, ids shuffled by one
    permutation whose first id is the poison block.  With ``num_blocks`` and
    ``sample_distinct``: one sample without replacement of (needed + 1)
    distinct ids from ``num_blocks`` (the extra one is the poison block).
    """
    need = [(int(s) + block_size - 1) // block_size for s in seq_lens]
    total = sum(need)
    if num_blocks is None:
        nb = total + 1
        ids = rng.permutation(nb)
    else:
        nb = int(num_blocks)
        if total + 1 > nb:
            raise ValueError("pool too small for the batch")
        ids = rng.choice(nb, size=total + 1, replace=False) if sample_distinct \
            else rng.permutation(nb)[: total + 1]
    poison = int(ids[0])
    max_blocks = max(1, max(need) if need else 1)
    table = np.full((len(seq_lens), max_blocks), poison, dtype=np.int32)
    owned = []
    cur = 1
    for r, n in enumerate(need):
        table[r, :n] = ids[cur:cur + n]
        owned.append(ids[cur:cur + n])
        cur += n
    return table, poison, nb, owned


def make_gqa(seed: int, q_lens, seq_lens, num_q_heads: int, num_kv_heads: int,
             head_dim: int = 128, block_size: int = 16, dtype: str = BF16,
             scale: float | None = None, num_blocks: int | None = None,
             sample_distinct: bool = False, name: str = "gqa",
             k_scale: float = 0.25, v_scale: float = 0.5) -> GqaBatch:
    """A paged GQA batch: request r has seq_lens[r] keys, the last q_lens[r] new.

    ``seed`` is an int or an already-advanced numpy Generator.  With dtype
    FP8 the cache holds E4M3 codes (uniform over the finite codes of
    magnitude <= 8, NaN 0x7F where nothing is stored) read with k_scale /
    v_scale; q and the new k / v rows are bf16 N(0,1)."""
    rng = seed if isinstance(seed, np.random.Generator) else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if np.any(q_lens > seq_lens) or np.any(q_lens < 0):
        raise ValueError("need 0 <= q_len <= seq_len")
    table, poison, nb, owned = _allocate_tables(rng, seq_lens, block_size,
                                                num_blocks, sample_distinct)
    T = int(q_lens.sum())
    qsl = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    row_dtype = BF16 if dtype == FP8 else dtype
    q = _normal(rng, (T, num_q_heads, head_dim), row_dtype)
    k_new = _normal(rng, (T, num_kv_heads, head_dim), row_dtype)
    v_new = _normal(rng, (T, num_kv_heads, head_dim), row_dtype)
    slots = np.empty(T, dtype=np.int64)
    valid = np.zeros((nb, block_size), dtype=bool)
    for r in range(len(seq_lens)):
        S, L = int(seq_lens[r]), int(q_lens[r])
        ctx = S - L
        pos = np.arange(S)
        blk = table[r, pos // block_size].astype(np.int64)
        off = pos % block_size
        valid[blk[:ctx], off[:ctx]] = True
        slots[qsl[r]:qsl[r + 1]] = blk[ctx:] * block_size + off[ctx:]
    cache = _fill_pool(rng, (nb, 2, block_size, num_kv_heads, head_dim), dtype)
    inval = ~valid
    cache[:, 0][inval] = _nan(dtype)
    cache[:, 1][inval] = _nan(dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    meta = {"k_scale": float(k_scale), "v_scale": float(v_scale)} if dtype == FP8 else {}
    return GqaBatch(name=name, dtype=dtype, q=q, k_new=k_new, v_new=v_new,
                    cache=cache, block_table=table, slot_mapping=slots,
                    query_start_loc=qsl, seq_lens=seq_lens.astype(np.int32),
                    scale=float(scale), block_size=block_size,
                    poison_block=poison, meta=meta)


def make_mla(seed: int, seq_lens, num_heads: int = 128, kv_lora_rank: int = 512,
             rope_dim: int = 64, block_size: int = 64, scale: float | None = None,
             name: str = "mla", cache_dtype: str = BF16, kv_scale: float = 0.25) -> MlaBatch:
    """An MLA decode batch: one new latent row per request at its last position.

    The default scale 1/sqrt(192) is that of a 128 + 64 query/key head.  With
    cache_dtype FP8 the cache holds E4M3 codes (as ``make_gqa``'s FP8 pool)
    read with one scale, kv_scale; the queries and new rows stay bf16."""
    rng = seed if isinstance(seed, np.random.Generator) else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if np.any(seq_lens < 1):
        raise ValueError("decode needs seq_len >= 1")
    table, poison, nb, owned = _allocate_tables(rng, seq_lens, block_size)
    B = len(seq_lens)
    q_nope = _normal(rng, (B, num_heads, kv_lora_rank), BF16)
    q_pe = _normal(rng, (B, num_heads, rope_dim), BF16)
    kv_c = _normal(rng, (B, kv_lora_rank), BF16)
    k_pe = _normal(rng, (B, rope_dim), BF16)
    valid = np.zeros((nb, block_size), dtype=bool)
    slots = np.empty(B, dtype=np.int64)
    for r in range(B):
        S = int(seq_lens[r])
        pos = np.arange(S)
        blk = table[r, pos // block_size].astype(np.int64)
        off = pos % block_size
        valid[blk[:S - 1], off[:S - 1]] = True
        slots[r] = blk[S - 1] * block_size + off[S - 1]
    cache = _fill_pool(rng, (nb, block_size, kv_lora_rank + rope_dim), cache_dtype)
    cache[~valid] = _nan(cache_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(192.0)
    meta = {"cache_dtype": FP8, "kv_scale": float(kv_scale)} if cache_dtype == FP8 else {}
    return MlaBatch(name=name, q_nope=q_nope, q_pe=q_pe, kv_c_new=kv_c,
                    k_pe_new=k_pe, cache=cache, block_table=table,
                    slot_mapping=slots, seq_lens=seq_lens.astype(np.int32),
                    scale=float(scale), block_size=block_size,
                    poison_block=poison, meta=meta)


@dataclass
class MlaPrefillBatch:
    """Inputs of one MLA prefill call (multi-head form).

    q [T, H, 192] (q_nope 128 | q_pe 64); kv_c_new [T, 512], k_pe_new [T, 64];
    cache [nb, bs, 576] latent rows (prior context only); w_kv_b [H * 256, 512]
    (per head: 128 key rows, 128 value rows); block_table [N, max_blocks];
    slot_mapping [T]; query_start_loc [N + 1]; seq_lens [N].  bf16.
    """
    name: str
    q: np.ndarray
    kv_c_new: np.ndarray
    k_pe_new: np.ndarray
    cache: np.ndarray
    w_kv_b: np.ndarray
    block_table: np.ndarray
    slot_mapping: np.ndarray
    query_start_loc: np.ndarray
    seq_lens: np.ndarray
    scale: float
    block_size: int
    poison_block: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self): return len(self.seq_lens)
    @property
    def num_tokens(self): return self.q.shape[0]
    @property
    def num_heads(self): return self.q.shape[1]
    @property
    def q_lens(self): return np.diff(self.query_start_loc)
    @property
    def max_query_len(self): return int(self.q_lens.max()) if len(self.seq_lens) else 0
    @property
    def total_keys(self): return int(self.seq_lens.astype(np.int64).sum())


def make_mla_prefill(seed, q_lens, seq_lens, num_heads: int = 16, block_size: int = 64,
                     scale: float | None = None, name: str = "mla_prefill") -> MlaPrefillBatch:
    """An MLA prefill batch: request r has seq_lens[r] keys, the last q_lens[r]
    new (their latent rows written by the call).  Latent rows, queries and new
    rows are bf16 N(0,1); kv_b_proj's weight is bf16 N(0,1) / 16 (a power of
    two, so the scaling is exact), which gives projected keys and values of
    variance 2.  Scale 1/sqrt(192) by default."""
    rng = seed if isinstance(seed, np.random.Generator) else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if np.any(q_lens > seq_lens) or np.any(q_lens < 0):
        raise ValueError("need 0 <= q_len <= seq_len")
    table, poison, nb, owned = _allocate_tables(rng, seq_lens, block_size)
    T = int(q_lens.sum())
    qsl = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    q = _normal(rng, (T, num_heads, 192), BF16)
    kv_c = _normal(rng, (T, 512), BF16)
    k_pe = _normal(rng, (T, 64), BF16)
    w = _normal(rng, (num_heads * 256, 512), BF16)
    w = f32_to_bf16_bits(bf16_bits_to_f32(w) / 16.0)
    valid = np.zeros((nb, block_size), dtype=bool)
    slots = np.empty(T, dtype=np.int64)
    for r in range(len(seq_lens)):
        S, L = int(seq_lens[r]), int(q_lens[r])
        pos = np.arange(S)
        blk = table[r, pos // block_size].astype(np.int64)
        off = pos % block_size
        valid[blk[:S - L], off[:S - L]] = True
        slots[qsl[r]:qsl[r + 1]] = blk[S - L:] * block_size + off[S - L:]
    cache = _fill_pool(rng, (nb, block_size, 576), BF16)
    cache[~valid] = NAN_BF16
    if scale is None:
        scale = 1.0 / math.sqrt(192.0)
    return MlaPrefillBatch(name=name, q=q, kv_c_new=kv_c, k_pe_new=k_pe, cache=cache, w_kv_b=w,
                           block_table=table, slot_mapping=slots, query_start_loc=qsl,
                           seq_lens=seq_lens.astype(np.int32), scale=float(scale),
                           block_size=block_size, poison_block=poison)


MLA_PREFILL = "mla_prefill_bf16"


def mla_prefill_batch(seed: int = 1010, batch: int = 16, num_heads: int = 16) -> MlaPrefillBatch:
    """The chunked-prefill distribution (16 requests, chunk ~ U{64..2048} new
    queries over context ~ U{0..4096}) for MLA: 16 heads (one GPU's share of
    128 heads split over 8), kv_lora_rank 512 + rope 64 latent rows, qk 192 /
    v 128 per head, block 64, bf16, causal."""
    rng = np.random.default_rng(seed)
    L = rng.integers(64, 2048, size=batch, endpoint=True)
    C = rng.integers(0, 4096, size=batch, endpoint=True)
    return make_mla_prefill(rng, L, C + L, num_heads, 64, name=MLA_PREFILL)


def mla_prefill_flops(b: MlaPrefillBatch) -> dict:
    """Projection: 2 x 512 x 256 per key and head; attention: 2 x (192 + 128)
    per visible (query, key) pair and head."""
    proj = 2 * 512 * 256 * b.num_heads * b.total_keys
    pairs = 0
    for L, S in zip(b.q_lens, b.seq_lens):
        L, S = int(L), int(S)
        pairs += L * (S - L) + L * (L + 1) // 2
    attn = 2 * (192 + 128) * b.num_heads * pairs
    return {"projection": proj, "attention": attn, "total": proj + attn}


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------

WORKLOADS = {
    0: "tiny_gqa_decode_fp32",
    1: "llama3_8b_gqa_decode_bf16",
    2: "chunked_prefill_varlen_bf16",
    3: "long_context_split_kv_decode_bf16",
    4: "mla_latent_decode_bf16",
}
MIXED = "mixed_prefill_decode_bf16"
CASCADE = "cascade_shared_prefix_decode_bf16"


def tiny_decode() -> GqaBatch:
    """3 requests (128, 1024, 4096 keys), 8 q / 2 kv heads, d=128, block 16,
    fp32, a 400-block pool; tables are one distinct sample of the pool."""
    b = make_gqa(1001, [1, 1, 1], [128, 1024, 4096], 8, 2, 128, 16, F32,
                 num_blocks=400, sample_distinct=True, name=WORKLOADS[0])
    return b


def llama_decode(seed: int = 1002, batch: int = 64) -> GqaBatch:
    """64 requests, seq_len ~ U{512..8192}, 32 q / 8 kv heads, d=128, bf16."""
    rng = np.random.default_rng(seed)
    seq = rng.integers(512, 8192, size=batch, endpoint=True)
    return make_gqa(rng, np.ones(batch, dtype=np.int64), seq, 32, 8, 128, 16,
                    BF16, name=WORKLOADS[1])


IDENTITY_DECODE = "llama3_8b_gqa_decode_bf16_identity_table"


def identity_layout(b: GqaBatch, name: str | None = None) -> GqaBatch:
    """The same batch with the pool's blocks renumbered so that request r's
    pages are consecutive physical blocks in logical order (an identity-like
    block table, requests one after another, the poison block last).  Every
    byte the attention reads is the same; only where the pages sit changes
    ("Attention Backends", Try it: the identity table gives the same result
    as a shuffled one)."""
    nb, bs = b.cache.shape[0], b.block_size
    need = (b.seq_lens.astype(np.int64) + bs - 1) // bs
    perm = np.full(nb, -1, dtype=np.int64)      # new id of old block b
    nxt = 0
    for r, n in enumerate(need):
        for old in b.block_table[r, :n]:
            perm[int(old)] = nxt
            nxt += 1
    rest = np.flatnonzero(perm < 0)
    perm[rest] = np.arange(nxt, nxt + len(rest))
    cache = np.empty_like(b.cache)
    cache[perm] = b.cache
    table = perm[b.block_table].astype(np.int32)
    slots = perm[b.slot_mapping // bs] * bs + b.slot_mapping % bs
    return GqaBatch(name=name or b.name, dtype=b.dtype, q=b.q, k_new=b.k_new, v_new=b.v_new,
                    cache=cache, block_table=table, slot_mapping=slots,
                    query_start_loc=b.query_start_loc, seq_lens=b.seq_lens, scale=b.scale,
                    block_size=bs, poison_block=int(perm[b.poison_block]), meta=dict(b.meta))


FP8_DECODE = "llama3_8b_gqa_decode_fp8kv"
FP8_MLA = "mla_latent_decode_fp8kv"
FP8_PREFILL = "chunked_prefill_varlen_fp8kv"


def chunked_prefill_fp8(seed: int = 1011, batch: int = 16) -> GqaBatch:
    """The chunked-prefill shape (16 requests, chunk U{64..2048} over context
    U{0..4096}, 32 q / 8 kv heads, d=128, block 16, causal) over an FP8
    cache, k_scale 0.25, v_scale 0.5."""
    rng = np.random.default_rng(seed)
    L = rng.integers(64, 2048, size=batch, endpoint=True)
    C = rng.integers(0, 4096, size=batch, endpoint=True)
    return make_gqa(rng, L, C + L, 32, 8, 128, 16, FP8, name=FP8_PREFILL, k_scale=0.25,
                    v_scale=0.5)


def mla_decode_fp8_batch(seed: int = 1009, batch: int = 128) -> MlaBatch:
    """The MLA decode shape (128 requests, seq_len ~ U{1024..8192}, 128 heads,
    512 + 64 latent row, block 64, scale 1/sqrt(192)) over an FP8 latent cache
    with kv_scale 0.25."""
    rng = np.random.default_rng(seed)
    seq = rng.integers(1024, 8192, size=batch, endpoint=True)
    return make_mla(rng, seq, 128, 512, 64, 64, 1.0 / math.sqrt(192), name=FP8_MLA,
                    cache_dtype=FP8, kv_scale=0.25)


def llama_decode_fp8(seed: int = 1008, batch: int = 64) -> GqaBatch:
    """The headline decode shape (64 requests, seq_len ~ U{512..8192}, 32 q /
    8 kv heads, d=128, block 16) over an FP8 (E4M3) cache, k_scale 0.25,
    v_scale 0.5; q and the new rows bf16."""
    rng = np.random.default_rng(seed)
    seq = rng.integers(512, 8192, size=batch, endpoint=True)
    return make_gqa(rng, np.ones(batch, dtype=np.int64), seq, 32, 8, 128, 16, FP8,
                    name=FP8_DECODE, k_scale=0.25, v_scale=0.5)


def chunked_prefill(seed: int = 1003, batch: int = 16) -> GqaBatch:
    """16 requests, chunk ~ U{64..2048} new queries over context ~ U{0..4096},
    32 q / 8 kv heads, d=128, bf16, block 16, causal within the chunk."""
    rng = np.random.default_rng(seed)
    L = rng.integers(64, 2048, size=batch, endpoint=True)
    C = rng.integers(0, 4096, size=batch, endpoint=True)
    return make_gqa(rng, L, C + L, 32, 8, 128, 16, BF16, name=WORKLOADS[2])


def long_context_decode(seed: int = 1004, batch: int = 4, seq_len: int = 131072) -> GqaBatch:
    """4 requests of 131072 keys, 64 q / 8 kv heads, d=128, bf16, block 16."""
    return make_gqa(seed, np.ones(batch, dtype=np.int64),
                    np.full(batch, seq_len), 64, 8, 128, 16, BF16,
                    name=WORKLOADS[3])


def mla_decode_batch(seed: int = 1005, batch: int = 128) -> MlaBatch:
    """128 requests, seq_len ~ U{1024..8192}, 128 heads, 512 + 64 latent row,
    block 64, scale 1/sqrt(192)."""
    rng = np.random.default_rng(seed)
    seq = rng.integers(1024, 8192, size=batch, endpoint=True)
    return make_mla(rng, seq, 128, 512, 64, 64, 1.0 / math.sqrt(192),
                    name=WORKLOADS[4])


def mixed_batch(seed: int = 1006, decode: int = 64, prefill: int = 4) -> GqaBatch:
    """A serving step that mixes both phases, decode requests first: 64
    decode requests (seq_len ~ U{512..8192}) then 4 prefill chunks (chunk ~
    U{64..2048} over context ~ U{0..4096}); 32 q / 8 kv heads, d=128, bf16,
    block 16 -- the decode and chunked-prefill workloads' distributions in
    one batch."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(512, 8192, size=decode, endpoint=True)
    L = rng.integers(64, 2048, size=prefill, endpoint=True)
    C = rng.integers(0, 4096, size=prefill, endpoint=True)
    q_lens = np.concatenate([np.ones(decode, dtype=np.int64), L])
    seq = np.concatenate([dec, C + L])
    return make_gqa(rng, q_lens, seq, 32, 8, 128, 16, BF16, name=MIXED)


def share_prefix(b: GqaBatch, prefix_blocks: int, name: str | None = None) -> GqaBatch:
    """Make every request start with request 0's first ``prefix_blocks``
    pages (a common prefix: the same physical pages, hence the same keys and
    values).  Each other request's own first pages are left unused and
    filled with NaN, so reading them shows.  Modifies ``b`` in place (its
    tables and pool) and returns it.  Every request's new tokens must lie
    after the prefix."""
    P = int(prefix_blocks)
    Lp = P * b.block_size
    if np.any(b.seq_lens.astype(np.int64) - b.q_lens < Lp):
        raise ValueError("every request's queries must follow the shared prefix")
    if P > 0 and b.num_seqs > 1:
        orphan = b.block_table[1:, :P].ravel()
        b.cache[orphan] = _nan(b.dtype)
        b.block_table[1:, :P] = b.block_table[0, :P]
    b.meta["prefix_blocks"] = P
    if name:
        b.name = name
    return b


def cascade_batch(seed: int = 1007, batch: int = 64, prefix_len: int = 4096) -> GqaBatch:
    """64 decode requests that share a 4096-token prefix (256 pages of 16,
    a common system prompt) followed by their own U{512..4096} tokens; 32 q /
    8 kv heads, d=128, bf16."""
    rng = np.random.default_rng(seed)
    own = rng.integers(512, 4096, size=batch, endpoint=True)
    b = make_gqa(rng, np.ones(batch, dtype=np.int64), prefix_len + own, 32, 8, 128, 16, BF16)
    return share_prefix(b, prefix_len // 16, name=CASCADE)


# --------------------------------------------------------------------------
# algorithmic work of a call (what the measurement is priced against)
# --------------------------------------------------------------------------

def gqa_bytes(b: GqaBatch, write: bool = True) -> dict:
    """Algorithmic HBM bytes of write + attention over a GQA batch.

    kv: every visible key and value row read once (all KV heads); q, out:
    once each; lse: fp32; write: new k/v read once and stored once; meta:
    block-table entries walked, seq_lens, query_start_loc, slot_mapping.
    Split-KV partials are implementation overhead and not counted.
    """
    e = b.elem_bytes
    row = b.num_kv_heads * b.head_dim * b.cache_elem_bytes
    kv = int(np.sum(b.seq_lens)) * row * 2
    q = b.q.size * e
    out = b.q.size * e
    lse = b.q.shape[0] * b.q.shape[1] * 4
    wr = (b.k_new.size + b.v_new.size) * (e + b.cache_elem_bytes) if write else 0
    nblk = int(np.sum((b.seq_lens.astype(np.int64) + b.block_size - 1) // b.block_size))
    meta = nblk * 4 + b.num_seqs * 8 + (b.num_tokens * 8 if write else 0)
    return {"kv": kv, "q": q, "out": out, "lse": lse, "write": wr, "meta": meta,
            "total": kv + q + out + lse + wr + meta}


def gqa_flops(b: GqaBatch, causal: bool = True) -> int:
    """2 flops per multiply-add of QK^T and PV over visible (query, key) pairs."""
    pairs = 0
    for L, S in zip(b.q_lens, b.seq_lens):
        L, S = int(L), int(S)
        pairs += (L * (S - L) + L * (L + 1) // 2) if causal else L * S
    return 2 * pairs * b.num_q_heads * (b.head_dim + b.head_dim)


def mla_bytes(b: MlaBatch, write: bool = True) -> dict:
    """Algorithmic bytes of MLA write + decode: each latent row read once."""
    rowb = (b.kv_lora_rank + b.rope_dim) * b.cache_elem_bytes
    kv = int(np.sum(b.seq_lens)) * rowb
    q = (b.q_nope.size + b.q_pe.size) * 2
    out = b.num_seqs * b.num_heads * b.kv_lora_rank * 2
    lse = b.num_seqs * b.num_heads * 4
    wr = (b.kv_c_new.size + b.k_pe_new.size) * (2 + b.cache_elem_bytes) if write else 0
    nblk = int(np.sum((b.seq_lens.astype(np.int64) + b.block_size - 1) // b.block_size))
    meta = nblk * 4 + b.num_seqs * 4 + (b.num_seqs * 8 if write else 0)
    return {"kv": kv, "q": q, "out": out, "lse": lse, "write": wr, "meta": meta,
            "total": kv + q + out + lse + wr + meta}


def mla_flops(b: MlaBatch) -> int:
    """2 flops per multiply-add: (R+P) for QK^T plus R for PV, per key per head."""
    return 2 * int(np.sum(b.seq_lens)) * b.num_heads * (2 * b.kv_lora_rank + b.rope_dim)
