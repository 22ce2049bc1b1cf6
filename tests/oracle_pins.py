"""Pins that tie the float64 oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages print, with a closed form, with an independent library routine
(torch's scaled_dot_product_attention / logsumexp in float64), with a
pure-Python brute force on tiny inputs, or with an invariant the pages state.
``test_oracle_pins.py`` runs every pin; ``test_oracle_mutations.py`` plants
plausible mistakes in the oracle and checks that some pin catches each one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle.pa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# storage and index pins
# --------------------------------------------------------------------------

def pin_bf16_decoding():
    """IEEE encodings: bf16 is the top half of an fp32 (textbook values)."""
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3E80, 0x4049, 0x7F80, 0xFF80],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 0.25, 3.140625, math.inf, -math.inf]
    got = O.bf16_bits_to_f64(bits)
    assert list(got) == want, got
    assert np.signbit(got[3])


def _paged_program_arrays():
    """The page's program geometry (block size, dim, pool, table, length) from
    the golden file, with this project's own seeded keys, values and query."""
    g = _golden("paged_program.json")
    rng = _rng(29)
    n, dim = g["seqLen"], g["dim"]
    keys = rng.standard_normal((n, dim))
    vals = rng.standard_normal((n, dim))
    q = rng.standard_normal(dim)
    return g, keys, vals, q


def _paged_program_cache(g, keys, vals, table):
    """Store the sequence at the slots the page's formula gives."""
    bs, nblk, dim = g["blockSize"], g["numBlocks"], g["dim"]
    cache = np.zeros((nblk, 2, bs, 1, dim))
    slots = np.array([O.slot_of(table, p, bs) for p in range(len(keys))])
    cache = O.cache_write_kv(cache, keys[:, None, :], vals[:, None, :], slots)
    return cache, slots


def pin_paged_program_slots():
    """The slot ranges the page's program prints for blockTable {6, 1, 4}."""
    g, keys, vals, _ = _paged_program_arrays()
    table = np.array(g["blockTable"])
    cache, slots = _paged_program_cache(g, keys, vals, table)
    rng = g["slot_ranges_printed"]
    assert [int(slots[0]), int(slots[3])] == rng["positions 0-3"]
    assert [int(slots[4]), int(slots[7])] == rng["positions 4-7"]
    assert [int(slots[8]), int(slots[9])] == rng["positions 8-9"]
    # exactly slotsUsed of slotsTotal slots hold the sequence
    flatk = cache[:, 0, :, 0, :].reshape(-1, g["dim"])
    used = np.flatnonzero(np.any(flatk != 0, axis=1))
    assert len(used) == g["slots_used"] and flatk.shape[0] == g["slots_total"]
    assert sorted(used.tolist()) == sorted(slots.tolist())
    # the gather returns the contiguous arrays bit for bit
    k2, v2 = O.gather_kv(cache, table, len(keys))
    assert np.array_equal(k2[:, 0], keys) and np.array_equal(v2[:, 0], vals)


def pin_paged_program_identical():
    """Paged == contiguous, bit for bit, for the page's table and its Try-it
    tables; the contiguous result matches torch's float64 attention."""
    g, keys, vals, q = _paged_program_arrays()
    scale = 1.0 / math.sqrt(g["dim"])
    contiguous, lse_c = O.attention(q[None, None, :], keys[:, None, :], vals[:, None, :],
                                    scale, None)
    ref = _sdpa(q[None, None, :], keys[:, None, :], vals[:, None, :], scale, None)
    assert np.max(np.abs(contiguous - ref)) < 1e-14, (contiguous, ref)
    assert np.max(np.abs(lse_c - _torch_lse(q[None, None, :], keys[:, None, :], scale, None))) < 1e-14
    for table in [g["blockTable"]] + g["try_it_tables"]:
        table = np.array(table)
        cache, _ = _paged_program_cache(g, keys, vals, table)
        qsl = np.array([0, 1])
        out, lse = O.paged_attention(q[None, None, :], cache, table[None, :], qsl,
                                     np.array([g["seqLen"]]), scale, causal=True)
        assert np.array_equal(out, contiguous) == g["identical"], table
        assert np.array_equal(lse, lse_c)


def pin_num_kv_splits():
    """max_seq_len / 512 splits, capped at 2 x compute units (Triton/MLA page,
    關鍵檔案); the long-context workload's 131072 keys on 256 CUs give 256."""
    assert O.num_kv_splits(131072, 256) == 256
    assert O.num_kv_splits(4096, 256) == 8
    assert O.num_kv_splits(8192, 256) == 16
    assert O.num_kv_splits(10 ** 7, 256) == 512
    assert O.num_kv_splits(1000, 2) == 2
    assert O.num_kv_splits(10 ** 7, 2) == 4
    assert O.num_kv_splits(1, 256) == 1
    assert O.num_kv_splits(0, 256) == 1
    assert O.num_kv_splits(513, 256) == 2      # rounds up (reading)
    assert O.num_kv_splits(512, 256) == 1


def pin_cache_write_bytes():
    """Written slots hold the new rows bit for bit, K in half 0 and V in half
    1; every other byte is untouched; negative slots are skipped."""
    rng = _rng(7)
    nb, bs, H, D = 9, 16, 3, 8
    cache = rng.integers(0, 65536, size=(nb, 2, bs, H, D), dtype=np.uint16)
    T = 20
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[5] = -1
    k = rng.integers(0, 65536, size=(T, H, D), dtype=np.uint16)
    v = rng.integers(0, 65536, size=(T, H, D), dtype=np.uint16)
    out = O.cache_write_kv(cache, k, v, slots)
    flat_k = out[:, 0].reshape(nb * bs, H, D)
    flat_v = out[:, 1].reshape(nb * bs, H, D)
    touched = np.zeros(nb * bs, dtype=bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(flat_k[s], k[t]) and np.array_equal(flat_v[s], v[t])
        touched[s] = True
    ck = cache[:, 0].reshape(nb * bs, H, D)
    cv = cache[:, 1].reshape(nb * bs, H, D)
    assert np.array_equal(flat_k[~touched], ck[~touched])
    assert np.array_equal(flat_v[~touched], cv[~touched])
    # MLA row layout: kv_c then k_pe
    mc = rng.integers(0, 65536, size=(4, 8, 12), dtype=np.uint16)
    kvc = rng.integers(0, 65536, size=(2, 9), dtype=np.uint16)
    kpe = rng.integers(0, 65536, size=(2, 3), dtype=np.uint16)
    mo = O.cache_write_mla(mc, kvc, kpe, np.array([13, -1]))
    assert np.array_equal(mo[1, 5], np.concatenate([kvc[0], kpe[0]]))
    mo[1, 5] = mc[1, 5]
    assert np.array_equal(mo, mc)


# --------------------------------------------------------------------------
# merge pins
# --------------------------------------------------------------------------

def pin_fig5c_merge():
    """Figure 5c: 15 after block A, A's share 1/3 once B joins, merged 28.33."""
    g = _golden("fig5c_merge.json")
    V = np.array(g["V"], dtype=np.float64)
    a_idx, b_idx = g["block_A_keys"], g["block_B_keys"]
    for base in (-3.0, 0.0, 11.5):
        scores = np.array([base, base, base + math.log(2), base + math.log(2)])
        q = np.ones((1, 1, 1))
        keys = scores.reshape(4, 1, 1)
        vals = V.reshape(4, 1, 1)
        oA, lA = O.attention(q, keys[a_idx], vals[a_idx], 1.0, None)
        oB, lB = O.attention(q, keys[b_idx], vals[b_idx], 1.0, None)
        assert abs(oA[0, 0, 0] - g["output_after_A"]) < 1e-12
        out, lse = O.lse_merge(np.stack([oA[0, 0], oB[0, 0]])[None],
                               np.array([[lA[0, 0], lB[0, 0]]]))
        share = math.exp(lA[0, 0] - lse[0])
        assert abs(share - g["share_of_A_after_B"]) < 1e-12
        assert round(float(out[0, 0]), g["merged_printed_decimals"]) == g["merged_printed"]
        assert abs(out[0, 0] - 85.0 / 3.0) < 1e-12
        naive, nl = O.attention(q, keys, vals, 1.0, None)
        assert abs(naive[0, 0, 0] - out[0, 0]) < 1e-12 and abs(nl[0, 0] - lse[0]) < 1e-12


def pin_merge_edges():
    """-inf splits weigh nothing; all -inf gives out 0, lse -inf; one finite
    split passes through unchanged; merging is order independent."""
    o = np.array([[[1.0, 2.0], [5.0, 7.0], [9.0, 9.0]]])
    out, lse = O.lse_merge(o, np.array([[-math.inf, 0.25, -math.inf]]))
    assert np.array_equal(out[0], [5.0, 7.0]) and lse[0] == 0.25
    out, lse = O.lse_merge(o, np.full((1, 3), -math.inf))
    assert np.array_equal(out[0], [0.0, 0.0]) and lse[0] == -math.inf
    rng = _rng(3)
    oo = rng.standard_normal((2, 5, 4))
    ll = rng.standard_normal((2, 5)) * 3
    a, la = O.lse_merge(oo, ll)
    p = rng.permutation(5)
    b, lb = O.lse_merge(oo[:, p], ll[:, p])
    assert np.allclose(a, b, rtol=0, atol=1e-13) and np.allclose(la, lb, rtol=0, atol=1e-13)
    # lse of the merge is ln(sum exp(lse_s)) computed by numpy's logaddexp
    assert np.allclose(la, np.logaddexp.reduce(ll, axis=1), rtol=0, atol=1e-13)
    packed = np.concatenate([oo, ll[..., None]], axis=-1)
    c, lc = O.lse_merge_packed(packed)
    assert np.array_equal(c, a) and np.array_equal(lc, la)


# --------------------------------------------------------------------------
# attention pins
# --------------------------------------------------------------------------

def pin_closed_forms():
    """One key -> its value and its score; zero query -> mean of the visible
    values and lse = ln(#visible); equal keys -> mean of values."""
    rng = _rng(11)
    Hq, Hkv, D = 4, 2, 16
    q = rng.standard_normal((1, Hq, D))
    K = rng.standard_normal((1, Hkv, D))
    V = rng.standard_normal((1, Hkv, D))
    out, lse = O.attention(q, K, V, 0.3, 0)
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        assert np.array_equal(out[0, h], V[0, kv])
        assert abs(lse[0, h] - 0.3 * float(q[0, h] @ K[0, kv])) < 1e-12
    S = 37
    K = rng.standard_normal((S, Hkv, D))
    V = rng.standard_normal((S, Hkv, D))
    L = 5
    out, lse = O.attention(np.zeros((L, Hq, D)), K, V, 0.7, S - L)
    for i in range(L):
        nvis = S - L + i + 1
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            assert np.allclose(out[i, h], V[:nvis, kv].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[i, h] - math.log(nvis)) < 1e-13
    Keq = np.repeat(rng.standard_normal((1, Hkv, D)), S, axis=0)
    q = rng.standard_normal((1, Hq, D))
    out, _ = O.attention(q, Keq, V, 0.2, None)
    for h in range(Hq):
        assert np.allclose(out[0, h], V[:, h // 2].mean(axis=0), rtol=0, atol=1e-12)


def _sdpa(q, K, V, scale, mask):
    """torch scaled_dot_product_attention (float64, CPU) with GQA sharing."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, scale=scale, enable_gqa=(K.shape[1] != q.shape[1]))
    return o[0].numpy().transpose(1, 0, 2)


def _torch_lse(q, K, scale, mask):
    tq = torch.from_numpy(q)          # [L, Hq, D]
    tk = torch.from_numpy(K)          # [S, Hkv, D]
    g = q.shape[1] // K.shape[1]
    tk = tk.repeat_interleave(g, dim=1)
    z = torch.einsum("lhd,shd->hls", tq, tk) * scale
    if mask is not None:
        z = z.masked_fill(~torch.from_numpy(mask)[None], float("-inf"))
    return torch.logsumexp(z, dim=-1).numpy().T


def pin_torch_sdpa_gqa():
    """Random GQA, bottom-right causal and unmasked, against torch's float64
    scaled_dot_product_attention (repeat-interleaved KV heads) and logsumexp."""
    rng = _rng(5)
    for (L, S, Hq, Hkv, D, causal) in [(1, 50, 8, 2, 32, True), (7, 23, 6, 3, 16, True),
                                       (9, 9, 4, 4, 8, True), (5, 12, 8, 1, 24, False),
                                       (3, 40, 4, 2, 128, True)]:
        q = rng.standard_normal((L, Hq, D))
        K = rng.standard_normal((S, Hkv, D))
        V = rng.standard_normal((S, Hkv, D)) * 2 + 0.5
        scale = 1.0 / math.sqrt(D) * 1.3
        mask = None
        if causal:
            mask = np.arange(S)[None, :] <= (S - L + np.arange(L))[:, None]
        out, lse = O.attention(q, K, V, scale, (S - L) if causal else None)
        ref = _sdpa(q, K, V, scale, mask)
        assert np.max(np.abs(out - ref)) < 1e-12, np.max(np.abs(out - ref))
        assert np.max(np.abs(lse - _torch_lse(q, K, scale, mask))) < 1e-12


def pin_torch_sdpa_mla():
    """MLA: q = [q_nope | q_pe] over the full row, V = first R columns,
    against torch's float64 scaled_dot_product_attention with one KV head."""
    rng = _rng(9)
    B, H, R, P, bs = 2, 6, 16, 4, 8
    seq = np.array([19, 8])
    nb = 8
    cache = rng.standard_normal((nb, bs, R + P)).astype(np.float32)
    table = np.array([[3, 5, 0], [6, 1, 1]], dtype=np.int32)
    qn = rng.standard_normal((B, H, R)).astype(np.float32)
    qp = rng.standard_normal((B, H, P)).astype(np.float32)
    out, lse = O.mla_decode(qn, qp, cache, table, seq, 0.21)
    for r in range(B):
        rows = np.concatenate([cache[table[r, j]] for j in range(3)])[: seq[r]].astype(np.float64)
        q = np.concatenate([qn[r], qp[r]], axis=-1).astype(np.float64)[None]
        ref = _sdpa(q, rows[:, None, :], rows[:, None, :R], 0.21, None)
        assert np.max(np.abs(out[r] - ref[0])) < 1e-12
        assert np.max(np.abs(lse[r] - _torch_lse(q, rows[:, None, :], 0.21, None)[0])) < 1e-12


def pin_bruteforce_varlen():
    """Pure-Python scalar loops over a tiny paged varlen causal batch."""
    rng = _rng(13)
    bs, Hq, Hkv, D = 4, 4, 2, 3
    q_lens = [2, 1, 3]
    seq = [6, 1, 9]
    nb = 8
    cache = rng.standard_normal((nb, 2, bs, Hkv, D))
    table = np.array([[5, 2, 0], [7, 0, 0], [1, 3, 6]], dtype=np.int32)
    qsl = np.array([0, 2, 3, 6])
    T = 6
    q = rng.standard_normal((T, Hq, D))
    scale = 0.77
    out, lse = O.paged_attention(q, cache, table, qsl, np.array(seq), scale, causal=True)
    for r in range(3):
        L, S = q_lens[r], seq[r]
        for i in range(L):
            t = qsl[r] + i
            for h in range(Hq):
                kvh = h * Hkv // Hq
                sc = []
                for j in range(S - L + i + 1):
                    b, o = table[r][j // bs], j % bs
                    sc.append((scale * sum(q[t, h, d] * cache[b, 0, o, kvh, d] for d in range(D)),
                               [cache[b, 1, o, kvh, d] for d in range(D)]))
                mx = max(s for s, _ in sc)
                den = sum(math.exp(s - mx) for s, _ in sc)
                for d in range(D):
                    num = sum(math.exp(s - mx) * v[d] for s, v in sc)
                    assert abs(out[t, h, d] - num / den) < 1e-13
                assert abs(lse[t, h] - (mx + math.log(den))) < 1e-13


# --------------------------------------------------------------------------
# invariants the pages state
# --------------------------------------------------------------------------

def pin_split_merge_equals_unsplit():
    """Split-KV partials merged by LSE equal unsplit attention (第 1 章 §3.1:
    splitting adds parallelism, every key still takes part)."""
    rng = _rng(17)
    S, L, Hq, Hkv, D = 45, 3, 4, 2, 16
    q = rng.standard_normal((L, Hq, D))
    K = rng.standard_normal((S, Hkv, D)) * 2
    V = rng.standard_normal((S, Hkv, D))
    full, lfull = O.attention(q, K, V, 0.4, S - L)
    for cuts in ([0, 45], [0, 16, 45], [0, 7, 8, 30, 45], [0, 44, 45], list(range(0, 46, 5))):
        parts = [O.partial_attention(q, K, V, 0.4, lo, hi, S - L)
                 for lo, hi in zip(cuts[:-1], cuts[1:])]
        outs = np.stack([p[0] for p in parts], axis=2)       # [L, Hq, nsplit, D]
        lses = np.stack([p[1] for p in parts], axis=2)
        out, lse = O.lse_merge(outs, lses)
        assert np.max(np.abs(out - full)) < 1e-12 and np.max(np.abs(lse - lfull)) < 1e-12


def pin_block_permutation():
    """Moving physical blocks (and the tables with them) changes nothing, bit
    for bit ("Attention Backends", Try it)."""
    rng = _rng(19)
    bs, Hq, Hkv, D = 16, 8, 2, 32
    seq = np.array([70, 16, 33])
    need = (seq + bs - 1) // bs
    nb = int(need.sum()) + 2
    cache = rng.standard_normal((nb, 2, bs, Hkv, D))
    ids = rng.permutation(nb)
    table = np.zeros((3, need.max()), dtype=np.int32)
    c = 0
    for r in range(3):
        table[r, :need[r]] = ids[c:c + need[r]]
        c += need[r]
    q = rng.standard_normal((3, Hq, D))
    out, lse = O.paged_decode(q, cache, table, seq, 0.2)
    perm = rng.permutation(nb)                   # new home of block b is perm[b]
    cache2 = np.empty_like(cache)
    cache2[perm] = cache
    table2 = perm[table].astype(np.int32)
    out2, lse2 = O.paged_decode(q, cache2, table2, seq, 0.2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def pin_chunked_prefill():
    """A prompt attended in two chunks gives, for the second chunk's queries,
    the same rows as attending it in one shot; a decode step equals the last
    row of a prefill over the same keys."""
    rng = _rng(23)
    S, Hq, Hkv, D = 40, 4, 2, 16
    q = rng.standard_normal((S, Hq, D))
    K = rng.standard_normal((S, Hkv, D))
    V = rng.standard_normal((S, Hkv, D))
    one, l1 = O.attention(q, K, V, 0.3, 0)
    c = 25
    second, l2 = O.attention(q[c:], K, V, 0.3, c)
    assert np.max(np.abs(second - one[c:])) < 1e-13 and np.max(np.abs(l2 - l1[c:])) < 1e-13
    dec, ld = O.attention(q[-1:], K, V, 0.3, S - 1)
    assert np.max(np.abs(dec - one[-1:])) < 1e-13 and np.max(np.abs(ld - l1[-1:])) < 1e-13


# --------------------------------------------------------------------------
# FP8 (E4M3) cache pins
# --------------------------------------------------------------------------

def pin_fp8_e4m3_decoding():
    """Values the OCP E4M3 definition fixes, and torch's float8_e4m3fn
    decoding of all 256 codes (an independent library routine)."""
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in want.items():
        got = O.fp8_e4m3_to_f64(np.array([c], np.uint8))[0]
        assert got == v, (hex(c), got, v)
    assert np.signbit(O.fp8_e4m3_to_f64(np.array([0x80], np.uint8))[0])
    codes = np.arange(256, dtype=np.uint8)
    got = O.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def pin_fp8_e4m3_encoding():
    """Round to nearest with ties to the even code, saturation at 448, the
    exact round trip of every finite code, brute-force nearest, and torch's
    float8_e4m3fn conversion of in-range fp32 values."""
    f = lambda *xs: list(O.f32_to_fp8_e4m3(np.array(xs, np.float32)))
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): the even code;
    # 1.1875 halfway between 1.125 and 1.25 (0x3A): the even code again
    assert f(1.0625, 1.1875, -1.0625) == [0x38, 0x3A, 0xB8]
    assert f(500.0, -1e9, 464.0, 447.0) == [0x7E, 0xFE, 0x7E, 0x7E]
    assert f(2.0 ** -10, 2.0 ** -10 * 1.0001, 3 * 2.0 ** -10) == [0x00, 0x01, 0x02]
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = O.fp8_e4m3_to_f64(codes).astype(np.float32)
    assert np.array_equal(O.f32_to_fp8_e4m3(vals), codes)
    rng = _rng(77)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-11, 9, 20000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    got = O.f32_to_fp8_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref), int((got != ref).sum())
    table = O.fp8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    for xi, ci in zip(x[:300], got[:300]):
        d = np.abs(table - abs(float(xi)))
        assert d[int(ci) & 0x7F] == d.min()


def pin_fp8_cache_write():
    """New rows are stored as E4M3(x / scale), the quotient in fp32 (torch's
    float8_e4m3fn conversion of the same quotient), K with k_scale and V with
    v_scale, at the same slots as the bf16 write; the dequantised cache holds
    code * scale per plane."""
    rng = _rng(78)
    nb, bs, H, D, T = 6, 16, 2, 8, 5
    cache = np.zeros((nb, 2, bs, H, D), np.uint8)
    k = (rng.standard_normal((T, H, D)) * 3).astype(np.float32)
    v = (rng.standard_normal((T, H, D)) * 0.02).astype(np.float32)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    vb = (v.view(np.uint32) >> 16).astype(np.uint16)
    ks, vs = 0.05, 0.0003
    slots = np.array([3, 17, 40, -1, 95])
    out = O.cache_write_kv_fp8(cache, kb, vb, slots, ks, vs)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        blk, off = divmod(int(sl), bs)
        for plane, bits, sc in ((0, kb, ks), (1, vb, vs)):
            qf = torch.from_numpy((bits[t].astype(np.uint32) << 16).view(np.float32)) / torch.tensor(
                sc, dtype=torch.float32)
            want = qf.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(out[blk, plane, off], want), (t, plane)
    written = {divmod(int(sl), bs) for sl in slots if sl >= 0}
    for blk in range(nb):
        for off in range(bs):
            if (blk, off) not in written:
                assert not out[blk, :, off].any()
    deq = O.dequant_kv_cache(out, ks, vs)
    ref = torch.from_numpy(out).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(deq[:, 0], ref[:, 0] * ks) and np.array_equal(deq[:, 1], ref[:, 1] * vs)


# --------------------------------------------------------------------------
# MLA prefill (multi-head form) pins
# --------------------------------------------------------------------------

def _mla_small_ints(seed, S_list, H, R, P, dn, dv):
    """Latent rows, kv_b_proj and queries of small integers, so that every
    expanded key and value is an exact bf16 value (no rounding anywhere)."""
    rng = _rng(seed)
    bs = 16
    nb = sum(-(-S // bs) for S in S_list) + 1
    cache = np.zeros((nb, bs, R + P))
    table = np.zeros((len(S_list), max(-(-S // bs) for S in S_list)), np.int32)
    cur = 1
    for r, S in enumerate(S_list):
        n = -(-S // bs)
        table[r, :n] = np.arange(cur, cur + n)
        cur += n
    cache[1:] = rng.integers(-2, 3, size=(nb - 1, bs, R + P))
    w = rng.integers(-1, 2, size=(H, dn + dv, R)).astype(np.float64)
    to_bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return to_bits(cache), table, to_bits(w), rng


def pin_mla_prefill_equals_absorbed_decode():
    """The two formulations of MLA ("Attention Backends": prefill and decode
    use different formulations of the same mathematics): for one query per
    request, attention over the expanded keys [kv_c W_k | k_pe] and values
    kv_c W_v equals attention over the latent rows with the absorbed query
    [W_k q_nope | q_pe], its latent output projected by W_v."""
    H, R, P, dn, dv = 3, 16, 8, 4, 5
    S_list = [1, 7, 40]
    cache, table, w, rng = _mla_small_ints(81, S_list, H, R, P, dn, dv)
    B = len(S_list)
    q = rng.standard_normal((B, H, dn + P))
    qsl = np.arange(B + 1)
    sl = np.array(S_list)
    out, lse = O.mla_prefill(q, cache, w, table, qsl, sl, 0.3, qk_nope=dn)
    W = O.to_f64(w)
    q_lat = np.einsum("bhd,hdr->bhr", q[:, :, :dn], W[:, :dn, :])    # W_k^T q_nope per head
    lat_out, lse2 = O.mla_decode(q_lat, q[:, :, dn:], cache, table, sl, 0.3)
    out2 = np.einsum("bhr,hvr->bhv", lat_out, W[:, dn:, :])
    assert np.max(np.abs(out - out2)) < 1e-10 and np.max(np.abs(lse - lse2)) < 1e-10


def pin_mla_prefill_torch_sdpa():
    """A chunked request (context + causal chunk) against torch's
    scaled_dot_product_attention in float64 on keys and values expanded with
    torch.einsum, the causal mask bottom-right aligned."""
    H, R, P, dn, dv = 2, 16, 8, 4, 6
    S_list, L = [30], 9
    cache, table, w, rng = _mla_small_ints(82, S_list, H, R, P, dn, dv)
    q = rng.standard_normal((L, H, dn + P))
    out, lse = O.mla_prefill(q, cache, w, table, np.array([0, L]), np.array(S_list), 0.4, qk_nope=dn)
    S = S_list[0]
    rows = torch.from_numpy(O.gather_mla(cache, table[0], S))
    W = torch.from_numpy(O.to_f64(w))
    kv = torch.einsum("sr,hcr->shc", rows[:, :R], W)
    K = torch.cat([kv[:, :, :dn], rows[:, None, R:].expand(S, H, P)], dim=-1)
    V = kv[:, :, dn:]
    mask = torch.arange(S)[None, :] <= (S - L + torch.arange(L))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), K.permute(1, 0, 2), V.permute(1, 0, 2),
        attn_mask=mask, scale=0.4).permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


# --------------------------------------------------------------------------
# bf16 rounding of the projection output, FP8 latent cache
# --------------------------------------------------------------------------

def _bf16_grid():
    """Every finite bf16 value (positive and negative), sorted, with its bits."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = O.bf16_bits_to_f64(bits)
    ok = np.isfinite(vals)
    order = np.argsort(vals[ok], kind="stable")
    return vals[ok][order], bits[ok][order]


def _nearest_bf16_brute(x):
    """Nearest bf16 value by search over the whole grid; a tie goes to the
    value whose bit pattern is even (round half to even)."""
    grid, gbits = _bf16_grid()
    out = np.empty(len(x))
    for i, xi in enumerate(np.asarray(x, np.float64)):
        d = np.abs(grid - xi)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            even = [b for b in best if gbits[b] % 2 == 0 and grid[b] != 0.0]
            best = even if even else best
        out[i] = grid[best[0]]
    return out


def pin_round_bf16():
    """Round to nearest bf16, ties to even: brute-force search of the bf16
    grid on random float64 values over the normal range, the halfway cases
    1 + 2^-8 -> 1 and 1 + 3 * 2^-8 -> 1 + 2^-6 (both signs), and torch's
    bfloat16 conversion of float32-exact values (one rounding)."""
    f = lambda *xs: list(O._round_bf16(np.array(xs, np.float64)))
    assert f(1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), -(1 + 3 * 2.0 ** -8)) == \
        [1.0, 1 + 2.0 ** -6, -1.0, -(1 + 2.0 ** -6)]
    assert f(1 + 2.0 ** -8 + 2.0 ** -30, 0.0, 3.0, -0.5) == [1 + 2.0 ** -7, 0.0, 3.0, -0.5]
    rng = _rng(91)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000))
    assert np.array_equal(O._round_bf16(x), _nearest_bf16_brute(x))
    x32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O._round_bf16(x32.astype(np.float64)), ref)


def pin_mla_expand_rounding():
    """The expanded keys and values are the exact products W kv_c rounded to
    the nearest bf16 (brute-force grid search), the key's rope part is k_pe
    unchanged, on random (not integer) inputs where rounding happens."""
    rng = _rng(92)
    H, R, P, dn, dv, S = 2, 16, 4, 3, 5, 6
    to_bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    rows = O.to_f64(to_bits(rng.standard_normal((S, R + P))))
    w = to_bits(rng.standard_normal((H, dn + dv, R)) / 4)
    keys, vals = O.mla_expand(rows, w, dn)
    W = O.to_f64(w)
    exact = np.einsum("sr,hcr->shc", rows[:, :R], W)
    want = _nearest_bf16_brute(exact.ravel()).reshape(exact.shape)
    assert np.array_equal(keys[:, :, :dn], want[:, :, :dn])
    assert np.array_equal(vals, want[:, :, dn:])
    assert np.array_equal(keys[:, :, dn:], np.broadcast_to(rows[:, None, R:], (S, H, P)))
    assert not np.array_equal(want, exact)        # rounding did happen


def pin_fp8_mla_cache_write():
    """The FP8 latent write: both parts of the row (kv_c and k_pe) stored as
    E4M3(x / scale) with one scale for the row ("Triton 與 MLA", 資料流:
    v_scale = k_scale for the latent cache), the quotient in fp32 and
    converted by torch's float8_e4m3fn; the dequantised cache holds
    code * scale (torch's decoding of the codes)."""
    rng = _rng(93)
    nb, bs, R, P, T = 4, 16, 12, 4, 5
    cache = np.full((nb, bs, R + P), 0x7F, np.uint8)
    to_bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kvc = to_bits(rng.standard_normal((T, R)) * 3)
    kpe = to_bits(rng.standard_normal((T, P)) * 3)
    sc = 0.37
    slots = np.array([2, 21, -1, 40, 63])
    out = O.cache_write_mla_fp8(cache, kvc, kpe, slots, sc)

    def ref_codes(bits):
        f = torch.from_numpy((bits.astype(np.uint32) << 16).view(np.float32))
        return (f / torch.tensor(sc, dtype=torch.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        blk, off = divmod(int(sl), bs)
        assert np.array_equal(out[blk, off, :R], ref_codes(kvc[t])), t
        assert np.array_equal(out[blk, off, R:], ref_codes(kpe[t])), t
    written = {divmod(int(sl), bs) for sl in slots if sl >= 0}
    for blk in range(nb):
        for off in range(bs):
            if (blk, off) not in written:
                assert np.all(out[blk, off] == 0x7F)
    finite = out.copy()
    finite[finite == 0x7F] = 0
    deq = O.dequant_mla_cache(finite, sc)
    ref = torch.from_numpy(finite).view(torch.float8_e4m3fn).double().numpy() * sc
    assert np.array_equal(deq, ref)


ALL_PINS = [
    pin_bf16_decoding, pin_paged_program_slots, pin_paged_program_identical,
    pin_num_kv_splits, pin_cache_write_bytes, pin_fig5c_merge, pin_merge_edges,
    pin_closed_forms, pin_torch_sdpa_gqa, pin_torch_sdpa_mla,
    pin_bruteforce_varlen, pin_split_merge_equals_unsplit, pin_block_permutation,
    pin_chunked_prefill, pin_fp8_e4m3_decoding, pin_fp8_e4m3_encoding, pin_fp8_cache_write,
    pin_mla_prefill_equals_absorbed_decode, pin_mla_prefill_torch_sdpa,
    pin_round_bf16, pin_mla_expand_rounding, pin_fp8_mla_cache_write,
]
