"""The seeded generators: determinism and the structure the recipe promises."""
import numpy as np

import workloads as W


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def test_same_seed_same_bytes():
    a = W.make_gqa(5, [3, 1], [40, 17], 8, 2, 64, 16, W.BF16)
    b = W.make_gqa(5, [3, 1], [40, 17], 8, 2, 64, 16, W.BF16)
    for f in ("q", "k_new", "v_new", "cache", "block_table", "slot_mapping"):
        assert np.array_equal(_bits(getattr(a, f)), _bits(getattr(b, f))), f
    c = W.make_gqa(6, [3, 1], [40, 17], 8, 2, 64, 16, W.BF16)
    assert not np.array_equal(a.q, c.q)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, np.inf, 3.0e38], np.float32)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> 1 + 2^-6 ... even mantissa
    got = W.f32_to_bf16_bits(x)
    assert got[0] == 0x3F80 and got[1] == 0x3F80 and got[2] == 0x3F82
    assert got[3] == 0xC020 and got[4] == 0x7F80
    assert W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_gqa_structure():
    b = W.make_gqa(9, [4, 1, 7], [36, 1, 70], 8, 2, 32, 16, W.BF16)
    bs = b.block_size
    assert b.cache.shape[0] == sum((s + bs - 1) // bs for s in [36, 1, 70]) + 1
    seen = set()
    for r, (L, S) in enumerate(zip(b.q_lens, b.seq_lens)):
        nblk = (S + bs - 1) // bs
        row = b.block_table[r]
        assert np.all(row[nblk:] == b.poison_block)
        assert not (set(row[:nblk].tolist()) & seen)
        seen |= set(row[:nblk].tolist())
        for i in range(L):
            pos = S - L + i
            assert b.slot_mapping[b.query_start_loc[r] + i] == row[pos // bs] * bs + pos % bs
        # context slots finite, new-token slots and tails NaN
        for pos in range(nblk * bs):
            blk, off = row[pos // bs], pos % bs
            v = W.bf16_bits_to_f32(b.cache[blk, 0, off])
            assert np.all(np.isfinite(v)) == (pos < S - L)
    assert np.all(np.isnan(W.bf16_bits_to_f32(b.cache[b.poison_block])))


def test_mla_structure():
    b = W.make_mla(3, [65, 130], 4, 16, 8, 64)
    assert b.cache.shape == (2 + 3 + 1, 64, 24)
    for r, S in enumerate(b.seq_lens):
        p = S - 1
        assert b.slot_mapping[r] == b.block_table[r, p // 64] * 64 + p % 64


def test_named_workload_shapes():
    t = W.tiny_decode()
    assert t.q.dtype == np.float32 and t.cache.shape == (400, 2, 16, 2, 128)
    assert list(t.seq_lens) == [128, 1024, 4096]
    ids = t.block_table[t.block_table != t.poison_block]
    assert len(ids) == 8 + 64 + 256 and len(set(ids.tolist())) == len(ids)


def test_byte_and_flop_counts():
    b = W.make_gqa(1, [1, 1], [100, 300], 32, 8, 128, 16, W.BF16)
    by = W.gqa_bytes(b)
    assert by["kv"] == 400 * 8 * 128 * 2 * 2
    assert W.gqa_flops(b) == 2 * 400 * 32 * 256


def test_identity_layout_same_bytes_consecutive_pages():
    """The identity-like layout moves pages, not values: every request's pages
    are consecutive in logical order, and the oracle's result is unchanged
    bit for bit."""
    import oracle.pa_oracle as O
    b = W.make_gqa(3, [1, 1, 1], [40, 300, 17], 8, 2, 128, 16, W.BF16)
    c = W.identity_layout(b, "identity")
    bs = b.block_size
    cur = 0
    for r, S in enumerate(b.seq_lens):
        n = -(-int(S) // bs)
        assert list(c.block_table[r, :n]) == list(range(cur, cur + n))
        cur += n
    o1, l1 = O.paged_decode(b.q, O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping),
                            b.block_table, b.seq_lens, b.scale)
    o2, l2 = O.paged_decode(c.q, O.cache_write_kv(c.cache, c.k_new, c.v_new, c.slot_mapping),
                            c.block_table, c.seq_lens, c.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert sorted(c.cache.reshape(c.cache.shape[0], -1).view(np.uint16)[:, 0].tolist()) == \
        sorted(b.cache.reshape(b.cache.shape[0], -1).view(np.uint16)[:, 0].tolist())
