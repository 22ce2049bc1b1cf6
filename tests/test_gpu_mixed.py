"""GPU parity of a planned mixed prefill + decode batch (pa_plan_mixed +
pa_mixed_attention) against the oracle's varlen paged attention, which
covers both phases with one definition (a decode request is the case of one
query row).  Also: the run gives, bit for bit, what the two group calls
give on their own, one plan serves several layers, and every decode
schedule the plan can pick (one pass, splits, token-balanced ranges)."""
import math

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _plan(b, cus=0):
    return pa.plan_mixed(b.query_start_loc, b.seq_lens, b.num_q_heads, b.num_kv_heads,
                         b.head_dim, b.block_size, b.block_table.shape[1], cus)


def _run(b, plan, write=True, cache_t=None):
    cache_t = to_dev(b.cache) if cache_t is None else cache_t
    out, lse = pa.mixed_attention(
        plan, to_dev(b.q), cache_t, to_dev(b.block_table), to_dev(b.query_start_loc),
        to_dev(b.seq_lens), b.scale, k=to_dev(b.k_new) if write else None,
        v=to_dev(b.v_new) if write else None,
        slot_mapping=to_dev(b.slot_mapping) if write else None)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(b, requests=None):
    cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
    out, lse = O.paged_attention(b.q, cache, b.block_table, b.query_start_loc, b.seq_lens,
                                 b.scale, causal=True, requests=requests)
    return cache, out, lse


def _check_rows(b, out, lse, oref, lref, requests, what):
    for r in requests:
        a0, a1 = b.query_start_loc[r], b.query_start_loc[r + 1]
        check_close(out[a0:a1], oref[a0:a1], f"{what} request {r} out")
        check_lse(lse[a0:a1], lref[a0:a1], f"{what} request {r} lse")


CASES = [
    # name, q_lens, seq_lens, Hq, Hkv  (decode requests first; later ones mix)
    ("balanced_decode_and_chunks", [1] * 6 + [70, 1, 200, 0, 129],
     [900, 17, 5000, 1, 3000, 2500, 100, 3000, 250, 12, 129], 32, 8),
    ("one_pass_decode", [1, 1, 1, 64, 33], [40, 100, 7, 300, 33], 8, 2),
    ("split_decode_6_kv_heads", [1, 1, 300], [9000, 14000, 900], 12, 6),
    ("decode_only", [1] * 12, list(range(300, 6300, 500)), 16, 4),
    ("prefill_only", [2, 1, 1, 90], [2, 40, 1, 400], 8, 8),
    ("g1_long_context_decode", [1, 1, 257], [30000, 2, 300], 4, 4),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
def test_mixed_small(ci):
    name, ql, sl, hq, hkv = CASES[ci]
    say(f"mixed {name}")
    b = W.make_gqa(300 + ci, ql, sl, hq, hkv, 128, 16, W.BF16, scale=1.0 / math.sqrt(128))
    plan = _plan(b)
    cache_t, out, lse = _run(b, plan)
    cache_ref, oref, lref = _oracle(b)
    assert np.array_equal(bits(cache_t), cache_ref)
    _check_rows(b, out, lse, oref, lref, range(b.num_seqs), name)


def test_mixed_equals_its_two_groups():
    """Decode rows equal pa_decode's (automatic schedule) over the decode
    requests alone; prefill rows equal pa_prefill_varlen's over the rest."""
    say("mixed vs separate group calls")
    b = W.make_gqa(321, [1] * 5 + [150, 1, 40], [3000, 800, 9000, 20, 4000, 600, 50, 40], 32, 8,
                   128, 16, W.BF16)
    plan = _plan(b)
    nd = plan.num_decode
    assert nd == 5
    cache_t, out, lse = _run(b, plan)   # writes the new rows; the calls below reuse the cache
    bt, sl, qsl = to_dev(b.block_table), to_dev(b.seq_lens), to_dev(b.query_start_loc)
    q = to_dev(b.q)
    od, ld = pa.decode(q[:nd].contiguous(), cache_t, bt[:nd].contiguous(), sl[:nd].contiguous(),
                       plan.max_decode_seq_len, b.scale)
    op, lp = pa.prefill_varlen(q, cache_t, bt[nd:].contiguous(), qsl[nd:].contiguous(),
                               sl[nd:].contiguous(), plan.max_query_len, plan.max_seq_len, b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(out[:nd], to_f64(od))
    assert np.array_equal(lse[:nd], ld.cpu().numpy().astype(np.float64))
    assert np.array_equal(out[nd:], to_f64(op[nd:]))
    assert np.array_equal(lse[nd:], lp[nd:].cpu().numpy().astype(np.float64))


def test_one_plan_serves_every_layer():
    """The plan depends only on the lengths: three layers (own q, k, v and
    cache contents, same tables and lengths) run with one plan."""
    say("mixed plan reused across layers")
    q_lens, seq = [1, 1, 1, 1, 100, 37], [5000, 3000, 64, 7000, 700, 37]
    base = W.make_gqa(330, q_lens, seq, 32, 8, 128, 16, W.BF16)
    plan = _plan(base)
    for layer in range(3):
        rng = np.random.default_rng(400 + layer)
        b = W.make_gqa(rng, q_lens, seq, 32, 8, 128, 16, W.BF16)
        # same lengths; the generator may place pages differently, which the plan
        # does not depend on
        cache_t, out, lse = _run(b, plan)
        cache_ref, oref, lref = _oracle(b)
        assert np.array_equal(bits(cache_t), cache_ref)
        _check_rows(b, out, lse, oref, lref, range(b.num_seqs), f"layer {layer}")


def test_plan_for_other_compute_unit_counts():
    """A plan sized for another device's compute-unit count gives a valid
    (differently partitioned) run on this one."""
    say("mixed plan for 80 and 1024 compute units")
    b = W.make_gqa(340, [1] * 8 + [65], [6000, 300, 8000, 1, 4000, 2000, 7000, 90, 65], 32, 8,
                   128, 16, W.BF16)
    cache_ref, oref, lref = _oracle(b)
    for cus in (80, 1024):
        plan = _plan(b, cus)
        _, out, lse = _run(b, plan)
        _check_rows(b, out, lse, oref, lref, range(b.num_seqs), f"{cus} CUs")


def test_mixed_deterministic():
    say("mixed determinism")
    b = W.make_gqa(350, [1, 1, 1, 120], [4000, 9000, 30, 500], 16, 4, 128, 16, W.BF16)
    plan = _plan(b)
    _, o1, l1 = _run(b, plan)
    _, o2, l2 = _run(b, plan)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.fixture(scope="module")
def mixed():
    return W.mixed_batch()


def test_mixed_workload_full_size(mixed):
    """64 decode requests (512..8192 keys) + 4 prefill chunks (64..2048 over
    0..4096 keys of context), 32/8 heads: 16 sampled decode rows (the
    longest and shortest among them) and the shortest and longest chunk
    against the oracle, the cache bit-exact."""
    b = mixed
    plan = _plan(b)
    say(f"mixed full size: {plan}")
    assert plan.num_decode == 64
    cache_t, out, lse = _run(b, plan)
    assert np.all(np.isfinite(out))
    ql = b.q_lens[64:]
    dl = b.seq_lens[:64]
    pick = np.random.default_rng(7).choice(64, size=14, replace=False)
    reqs = [int(x) for x in pick] + [int(np.argmax(dl)), int(np.argmin(dl)),
                                     64 + int(np.argmax(ql)), 64 + int(np.argmin(ql))]
    cache_ref, oref, lref = _oracle(b, requests=sorted(set(reqs)))
    _check_rows(b, out, lse, oref, lref, sorted(set(reqs)), "mixed workload")
    assert np.array_equal(bits(cache_t), cache_ref)
