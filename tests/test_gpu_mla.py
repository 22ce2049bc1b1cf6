"""GPU parity of pa_mla_decode (latent write + MQA decode over [kv_c | k_pe]
rows, split partials merged by LSE) against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

# Units of work a request start counts for when the MLA decode cuts its
# token-balanced ranges (documented with pa_mla_decode_balanced).
MLA_RANGE_OVERHEAD = 5


def _run(b: W.MlaBatch, num_splits=0, write=True, fused_q=False):
    cache_t = to_dev(b.cache)
    if fused_q:
        q = to_dev(np.concatenate([b.q_nope, b.q_pe], axis=-1))
        qn, qp = q[..., :b.kv_lora_rank], q[..., b.kv_lora_rank:]
    else:
        qn, qp = to_dev(b.q_nope), to_dev(b.q_pe)
    out, lse = pa.mla_decode(qn, qp, cache_t, to_dev(b.block_table), to_dev(b.seq_lens),
                             b.max_seq_len, b.scale,
                             kv_c=to_dev(b.kv_c_new) if write else None,
                             k_pe=to_dev(b.k_pe_new) if write else None,
                             slot_mapping=to_dev(b.slot_mapping) if write else None,
                             num_splits=num_splits)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(b: W.MlaBatch, requests=None):
    cache = O.cache_write_mla(b.cache, b.kv_c_new, b.k_pe_new, b.slot_mapping)
    out, lse = O.mla_decode(b.q_nope, b.q_pe, cache, b.block_table, b.seq_lens, b.scale,
                            requests=requests)
    return cache, out, lse


CASES = [
    # name, seq_lens, heads, block_size
    ("ragged_h128_b64", [1, 31, 32, 33, 64, 65, 700], 128, 64),
    ("h16_b16", [5, 100, 1000], 16, 16),
    ("h64_b64", [2000, 64], 64, 64),
    ("h48_b32", [77, 300], 48, 32),
    # page sizes that are multiples of 16 but not powers of two
    ("h128_b48", [47, 48, 49, 500, 1000], 128, 48),
    ("h32_b80", [79, 81, 1700], 32, 80),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_mla_small(ci, splits):
    name, seq, H, bs = CASES[ci]
    say(f"mla {name} splits={splits}")
    b = W.make_mla(300 + ci, seq, H, 512, 64, bs)
    cache_t, out, lse = _run(b, num_splits=splits, fused_q=(splits == 3))
    cache_ref, oref, lref = _oracle(b)
    assert np.array_equal(bits(cache_t), cache_ref)
    check_close(out, oref, f"{name} out")
    check_lse(lse, lref, f"{name} lse")


def test_mla_deterministic_and_permutation_invariant():
    say("mla determinism / block permutation")
    b = W.make_mla(12, [900, 64, 129], 32, 512, 64, 64)
    _, o1, l1 = _run(b, num_splits=2)
    _, o2, l2 = _run(b, num_splits=2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(4).permutation(b.num_blocks)
    cache2 = np.empty_like(b.cache)
    cache2[perm] = b.cache
    bb = W.MlaBatch(**{**b.__dict__, "cache": cache2,
                       "block_table": perm[b.block_table].astype(np.int32),
                       "slot_mapping": perm[b.slot_mapping // 64] * 64 + b.slot_mapping % 64})
    _, o3, l3 = _run(bb, num_splits=2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


@pytest.fixture(scope="module")
def mla_full():
    return W.mla_decode_batch()


def test_mla_full_size(mla_full):
    """128 requests x 128 heads, seq_len U{1024..8192}, block 64, scale
    1/sqrt(192); every request against the oracle."""
    b = mla_full
    say(f"mla full size max_seq_len={b.max_seq_len}")
    cache_t, out, lse = _run(b, num_splits=0)
    assert np.all(np.isfinite(out))
    cache_ref, oref, lref = _oracle(b)
    check_close(out, oref, "mla full out")
    check_lse(lse, lref, "mla full lse")
    assert np.array_equal(bits(cache_t), cache_ref)


def test_mla_two_stage_matches_one_call():
    say("mla two-stage")
    b = W.make_mla(13, [1500, 64, 700], 32, 512, 64, 64)
    cache_t, out1, lse1 = _run(b, num_splits=4)
    part = pa.mla_decode(to_dev(b.q_nope), to_dev(b.q_pe), cache_t, to_dev(b.block_table),
                         to_dev(b.seq_lens), b.max_seq_len, b.scale, num_splits=4,
                         stage1_only=True)
    out2, lse2 = pa.lse_merge(part, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert part.shape == (3, 32, 4, 513)
    assert np.array_equal(to_f64(out2), out1)
    assert np.array_equal(lse2.cpu().numpy().astype(np.float64), lse1)


# ------------------------------------------------- token-balanced schedule
def _run_balanced(b: W.MlaBatch, num_ranges, merge=True, seq_lens=None):
    sl = b.seq_lens if seq_lens is None else seq_lens
    cache = O.cache_write_mla(b.cache, b.kv_c_new, b.k_pe_new, b.slot_mapping)
    out, lse, ws, nr = pa.mla_decode_balanced(to_dev(b.q_nope), to_dev(b.q_pe), to_dev(cache),
                                              to_dev(b.block_table),
                                              to_dev(np.asarray(sl, dtype=np.int32)), b.scale,
                                              num_ranges=num_ranges, merge=merge)
    torch.cuda.synchronize()
    return cache, out, lse, ws, nr


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_ranges", [1, 2, 5, 40, 100000])
def test_mla_balanced_small(ci, num_ranges):
    name, seq, H, bs = CASES[ci]
    say(f"mla balanced {name} ranges={num_ranges}")
    b = W.make_mla(300 + ci, seq, H, 512, 64, bs)
    cache, out, lse, _, _ = _run_balanced(b, num_ranges)
    oref, lref = O.mla_decode(b.q_nope, b.q_pe, cache, b.block_table, b.seq_lens, b.scale)
    check_close(to_f64(out), oref, f"{name} out")
    check_lse(lse.cpu().numpy().astype(np.float64), lref, f"{name} lse")


@pytest.mark.parametrize("num_ranges", [3, 11])
def test_mla_balanced_segments_against_oracle(num_ranges):
    """Stage 1 alone: prefix sums exact, whole requests final, and every
    segment partial equal to the oracle's attention over that range's keys."""
    seq = [700, 33, 1, 2000, 64, 130]
    say(f"mla balanced segments ranges={num_ranges}")
    b = W.make_mla(14, seq, 32, 512, 64, 64)
    B, H = b.num_seqs, b.num_heads
    cache, out, lse, ws, nr_arg = _run_balanced(b, num_ranges, merge=False)
    # the MLA ranges count each request start as MLA_RANGE_OVERHEAD units of
    # work: request r is units [cu[r], cu[r + 1]), its chunks the last n_r
    n = [-(-s // 32) for s in seq]
    units = [k + MLA_RANGE_OVERHEAD if k else 0 for k in n]
    cu = np.concatenate([[0], np.cumsum(units)]).astype(np.int64)
    first = cu[:-1] + MLA_RANGE_OVERHEAD   # unit of each request's first chunk
    T = int(cu[-1])
    nr = min(num_ranges, T)
    ranges = [(j * T // nr, (j + 1) * T // nr) for j in range(nr)]
    wsn = ws.cpu().numpy()
    assert np.array_equal(wsn.view(np.int32)[: B + 1], cu)
    off = ((B + 1) * 4 + 255) // 256 * 256 // 4
    part = wsn[off: off + (nr_arg + B) * H * 516].reshape(nr_arg + B, H, 516)
    o1, l1 = to_f64(out), lse.cpu().numpy().astype(np.float64)
    oref, lref = O.mla_decode(b.q_nope, b.q_pe, cache, b.block_table, b.seq_lens, b.scale)
    n_split = 0
    for r in range(B):
        js = [j for j, (c0, c1) in enumerate(ranges) if c0 < cu[r + 1] and c1 > first[r]]
        if len(js) == 1:
            check_close(o1[r], oref[r], f"direct request {r}")
            check_lse(l1[r], lref[r], f"direct request {r}")
            continue
        n_split += 1
        rows = O.gather_mla(cache, b.block_table[r], seq[r])
        q = np.concatenate([O.to_f64(b.q_nope[r]), O.to_f64(b.q_pe[r])], axis=-1)[None]
        for j in js:
            c0, c1 = ranges[j]
            lo = (max(c0, first[r]) - first[r]) * 32
            hi = min((min(c1, cu[r + 1]) - first[r]) * 32, seq[r])
            po, pl = O.partial_attention(q, rows[:, None, :], rows[:, None, :512], b.scale, lo, hi,
                                         None)
            check_close(part[j + r, :, :512].astype(np.float64), po[0],
                        f"request {r} range {j} partial")
            check_lse(part[j + r, :, 512].astype(np.float64), pl[0], f"request {r} range {j} lse")
    assert n_split > 0
    pa.decode_balanced_merge(ws, B, H, 512, nr_arg, out, lse)
    torch.cuda.synchronize()
    check_close(to_f64(out), oref, "merged out")
    check_lse(lse.cpu().numpy().astype(np.float64), lref, "merged lse")


def test_mla_automatic_schedule_is_balanced():
    say("mla balanced vs automatic pa_mla_decode")
    b = W.make_mla(15, [1500, 64, 700, 3000], 64, 512, 64, 64)
    cache_t, out1, lse1 = _run(b, num_splits=0)
    out2, lse2, _, nr = pa.mla_decode_balanced(to_dev(b.q_nope), to_dev(b.q_pe), cache_t,
                                               to_dev(b.block_table), to_dev(b.seq_lens), b.scale)
    torch.cuda.synchronize()
    assert nr == pa.device_num_cus()
    assert np.array_equal(to_f64(out2), out1)
    assert np.array_equal(lse2.cpu().numpy().astype(np.float64), lse1)


def test_mla_balanced_requests_without_keys():
    say("mla balanced empty requests")
    b = W.make_mla(16, [300, 5, 900, 40], 16, 512, 64, 16)
    seq = np.array([300, 0, 900, 0], dtype=np.int32)
    for nr in (1, 4, 100):
        cache, out, lse, _, _ = _run_balanced(b, nr, seq_lens=seq)
        oref, lref = O.mla_decode(b.q_nope, b.q_pe, cache, b.block_table, seq, b.scale)
        o, l = to_f64(out), lse.cpu().numpy().astype(np.float64)
        assert np.all(o[[1, 3]] == 0) and np.all(np.isneginf(l[[1, 3]]))
        check_close(o, oref, f"ranges={nr} out")
        check_lse(l, lref, f"ranges={nr} lse")


# ------------------------------------------ latent head size 320 (rank 256)
CASES_320 = [
    # name, seq_lens, heads, block_size
    ("r256_ragged_h128", [1, 31, 32, 33, 64, 65, 700], 128, 64),
    ("r256_h16_b16", [5, 100, 1000], 16, 16),
    ("r256_h64_long", [3000, 2], 64, 64),
]


@pytest.mark.parametrize("ci", range(len(CASES_320)), ids=[c[0] for c in CASES_320])
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_mla_rank256_head320(ci, splits):
    """kv_lora_rank 256 + rope 64: the 320-element latent row, through the
    balanced schedule (splits 0), one pass and explicit splits."""
    name, seq, H, bs = CASES_320[ci]
    say(f"mla 320 {name} splits={splits}")
    b = W.make_mla(350 + ci, seq, H, 256, 64, bs, scale=1.0 / math.sqrt(192))
    cache_t, out, lse = _run(b, num_splits=splits)
    cache_ref, oref, lref = _oracle(b)
    assert np.array_equal(bits(cache_t), cache_ref)
    check_close(out, oref, f"{name} out")
    check_lse(lse, lref, f"{name} lse")


@pytest.mark.parametrize("num_ranges", [1, 7, 300])
def test_mla_rank256_balanced_ranges(num_ranges):
    say(f"mla 320 balanced ranges={num_ranges}")
    b = W.make_mla(360, [1, 900, 64, 2000, 33], 32, 256, 64, 64)
    cache, out, lse, _, _ = _run_balanced(b, num_ranges)
    oref, lref = O.mla_decode(b.q_nope, b.q_pe, cache, b.block_table, b.seq_lens, b.scale)
    check_close(to_f64(out), oref, "320 balanced out")
    check_lse(lse.cpu().numpy().astype(np.float64), lref, "320 balanced lse")
