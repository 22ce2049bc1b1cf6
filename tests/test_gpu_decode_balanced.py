"""GPU parity of the token-balanced decode schedule (pa_decode_balanced +
pa_decode_balanced_merge, and pa_decode's automatic schedule) against the
oracle.

The range partition is recomputed here from its definition -- the 32-token
chunks of all requests concatenated, range j = chunks [j T / nr, (j+1) T / nr),
nr = min(num_ranges, T) -- so that the chunk prefix sums are checked bit for
bit and every segment partial against the oracle's attention over the same
keys.  Outputs: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|; LSE within 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

CHUNK = 32
PART_ROW = 132


def _partition(seq_lens, num_ranges):
    n = [-(-int(s) // CHUNK) for s in seq_lens]
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    T = int(cu[-1])
    nr = min(num_ranges, T)
    ranges = [(j * T // nr, (j + 1) * T // nr) for j in range(nr)]
    return cu, nr, ranges


def _batch(seed, seq, hq, hkv, bs=16):
    b = W.make_gqa(seed, np.ones(len(seq), dtype=np.int64), seq, hq, hkv, 128, bs, W.BF16,
                   scale=0.9 / math.sqrt(128))
    # the balanced entry point reads the cache as is: store the new rows first
    cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
    return W.GqaBatch(**{**b.__dict__, "cache": cache})


def _run(b, num_ranges, merge=True, seq_lens=None):
    sl = b.seq_lens if seq_lens is None else seq_lens
    out, lse, ws, nr = pa.decode_balanced(to_dev(b.q), to_dev(b.cache), to_dev(b.block_table),
                                          to_dev(np.asarray(sl, dtype=np.int32)), b.scale,
                                          num_ranges=num_ranges, merge=merge)
    torch.cuda.synchronize()
    return out, lse, ws, nr


CASES = [
    # name, seq_lens, Hq, Hkv, block_size
    ("ragged_g4", [1, 15, 16, 17, 33, 100, 257, 700], 32, 8, 16),
    ("g8", [5, 64, 1000, 2049], 64, 8, 16),
    ("g1", [3, 40, 511, 513], 8, 8, 16),
    ("g2_block32", [31, 32, 33, 900], 4, 2, 32),
    ("hkv16_two_head_groups", [300, 1200, 2], 32, 16, 16),
    ("hkv1_g8_block64", [2000, 1, 77], 8, 1, 64),
    # page sizes that are multiples of 16 but not powers of two
    ("g4_block48", [47, 48, 49, 700, 1500], 32, 8, 48),
    ("g8_block80", [79, 81, 2000, 3], 64, 8, 80),
    ("hkv1_g4_block48", [95, 1, 1200], 4, 1, 48),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_ranges", [1, 2, 3, 7, 40, 100000])
def test_balanced_small(ci, num_ranges):
    name, seq, hq, hkv, bs = CASES[ci]
    say(f"balanced {name} ranges={num_ranges}")
    b = _batch(200 + ci, seq, hq, hkv, bs)
    out, lse, _, _ = _run(b, num_ranges)
    oref, lref = O.paged_decode(b.q, b.cache, b.block_table, b.seq_lens, b.scale)
    check_close(to_f64(out), oref, f"{name} out")
    check_lse(lse.cpu().numpy().astype(np.float64), lref, f"{name} lse")


@pytest.mark.parametrize("num_ranges", [3, 13, 64])
def test_balanced_segments_against_oracle(num_ranges):
    """Stage 1 alone: the prefix sums are exact, requests inside one range are
    final, and each segment partial is the oracle's attention over exactly the
    keys of that range; the merge then completes the rest."""
    seq = [700, 33, 1, 2000, 64, 65, 300]
    say(f"balanced segments ranges={num_ranges}")
    b = _batch(31, seq, 32, 8)
    B, Hq = b.num_seqs, b.num_q_heads
    out, lse, ws, nr_arg = _run(b, num_ranges, merge=False)
    cu, nr, ranges = _partition(seq, num_ranges)
    wsn = ws.cpu().numpy()
    cu_dev = wsn.view(np.int32)[: B + 1]
    assert np.array_equal(cu_dev, cu)
    off = ((B + 1) * 4 + 255) // 256 * 256 // 4
    part = wsn[off: off + (nr_arg + B) * Hq * PART_ROW].reshape(nr_arg + B, Hq, PART_ROW)
    o1 = to_f64(out)
    l1 = lse.cpu().numpy().astype(np.float64)
    oref, lref = O.paged_decode(b.q, b.cache, b.block_table, b.seq_lens, b.scale)
    n_split = 0
    for r in range(B):
        js = [j for j, (c0, c1) in enumerate(ranges) if c0 < cu[r + 1] and c1 > cu[r]]
        if len(js) == 1:
            check_close(o1[r], oref[r], f"direct request {r}")
            check_lse(l1[r], lref[r], f"direct request {r}")
            continue
        n_split += 1
        keys, vals = O.gather_kv(b.cache, b.block_table[r], seq[r])
        q = O.to_f64(b.q[r:r + 1])
        for j in js:
            c0, c1 = ranges[j]
            lo = (max(c0, cu[r]) - cu[r]) * CHUNK
            hi = min((min(c1, cu[r + 1]) - cu[r]) * CHUNK, seq[r])
            po, pl = O.partial_attention(q, keys, vals, b.scale, lo, hi, None)
            check_close(part[j + r, :, :128].astype(np.float64), po[0],
                        f"request {r} range {j} partial")
            check_lse(part[j + r, :, 128].astype(np.float64), pl[0], f"request {r} range {j} lse")
    assert n_split > 0
    pa.decode_balanced_merge(ws, B, Hq, 128, nr_arg, out, lse)
    torch.cuda.synchronize()
    check_close(to_f64(out), oref, "merged out")
    check_lse(lse.cpu().numpy().astype(np.float64), lref, "merged lse")


def test_automatic_schedule_is_balanced():
    """pa_decode with num_splits = 0 runs the write, then the balanced kernels
    with the device's range count: bit-identical to calling them directly."""
    say("balanced vs automatic pa_decode")
    b0 = W.make_gqa(41, np.ones(5, dtype=np.int64), [600, 5000, 1, 1300, 3000], 32, 8, 128, 16,
                    W.BF16)
    cache_t = to_dev(b0.cache)
    out1, lse1 = pa.decode(to_dev(b0.q), cache_t, to_dev(b0.block_table), to_dev(b0.seq_lens),
                           b0.max_seq_len, b0.scale, k=to_dev(b0.k_new), v=to_dev(b0.v_new),
                           slot_mapping=to_dev(b0.slot_mapping), num_splits=0)
    out2, lse2, _, nr = pa.decode_balanced(to_dev(b0.q), cache_t, to_dev(b0.block_table),
                                           to_dev(b0.seq_lens), b0.scale)
    torch.cuda.synchronize()
    assert nr == pa.decode_balanced_num_ranges(8, pa.device_num_cus())
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    cache = O.cache_write_kv(b0.cache, b0.k_new, b0.v_new, b0.slot_mapping)
    oref, lref = O.paged_decode(b0.q, cache, b0.block_table, b0.seq_lens, b0.scale)
    check_close(to_f64(out1), oref, "out")
    check_lse(lse1.cpu().numpy().astype(np.float64), lref, "lse")


def test_balanced_requests_without_keys():
    """A request with seq_len 0 gets out = 0 and lse = -inf; the others are
    unaffected (the oracle's convention for a query that sees no key)."""
    say("balanced empty requests")
    b = _batch(43, [300, 5, 900, 40], 16, 4)
    seq = np.array([300, 0, 900, 0], dtype=np.int32)
    for nr in (1, 5, 100):
        out, lse, _, _ = _run(b, nr, seq_lens=seq)
        oref, lref = O.paged_decode(b.q, b.cache, b.block_table, seq, b.scale)
        o = to_f64(out)
        l = lse.cpu().numpy().astype(np.float64)
        assert np.all(o[[1, 3]] == 0) and np.all(np.isneginf(l[[1, 3]]))
        check_close(o, oref, f"ranges={nr} out")
        check_lse(l, lref, f"ranges={nr} lse")


def test_balanced_deterministic_and_permutation_invariant():
    say("balanced determinism / block permutation")
    b = _batch(44, [300, 1, 1500, 16, 4000], 32, 8)
    o1, l1, _, _ = _run(b, 50)
    o2, l2, _, _ = _run(b, 50)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    perm = np.random.default_rng(6).permutation(b.num_blocks)
    cache2 = np.empty_like(b.cache)
    cache2[perm] = b.cache
    b2 = W.GqaBatch(**{**b.__dict__, "cache": cache2,
                       "block_table": perm[b.block_table].astype(np.int32)})
    o3, l3, _, _ = _run(b2, 50)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
