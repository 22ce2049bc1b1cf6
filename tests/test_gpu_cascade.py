"""GPU parity of cascade (shared-prefix) attention (pa_plan_cascade +
pa_cascade_attention) against the oracle's plain paged attention over the
whole keys: the prefix-once decomposition must give the ordinary result.
Covers decode-only and mixed batches, every supported GQA group, prefixes of
one page up to many key ranges with ragged tails, block size 32, several
compute-unit counts (different key-range cuts), plan reuse across layers,
the P = 0 degenerate case, and the full shared-prefix workload."""
import math

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _batch(seed, q_lens, own, prefix_blocks, hq, hkv, bs=16):
    seq = np.asarray(own) + prefix_blocks * bs
    b = W.make_gqa(seed, q_lens, seq, hq, hkv, 128, bs, W.BF16, scale=1.0 / math.sqrt(128))
    return W.share_prefix(b, prefix_blocks)


def _plan(b, prefix_blocks, cus=0):
    return pa.plan_cascade(b.query_start_loc, b.seq_lens, prefix_blocks, b.num_q_heads,
                           b.num_kv_heads, b.head_dim, b.block_size, b.block_table.shape[1], cus)


def _run(b, plan):
    cache_t = to_dev(b.cache)
    out, lse = pa.cascade_attention(
        plan, to_dev(b.q), cache_t, to_dev(b.block_table), to_dev(b.query_start_loc),
        to_dev(b.seq_lens), b.scale, k=to_dev(b.k_new), v=to_dev(b.v_new),
        slot_mapping=to_dev(b.slot_mapping))
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
    # name, q_lens, own keys (incl. the new ones), prefix pages, Hq, Hkv, block size
    ("decode_g4", [1] * 8, [1, 9, 300, 1000, 64, 2, 700, 129], 40, 32, 8, 16),
    ("mixed_g2", [1, 1, 1, 70, 200, 0], [5, 900, 33, 100, 260, 3], 17, 8, 4, 16),
    ("one_page_g8", [1, 1, 5], [40, 1, 5], 1, 8, 1, 16),
    ("long_prefix_g1", [1, 1, 1, 1], [10, 200, 3, 77], 300, 4, 4, 16),
    ("block32_ragged", [1, 1, 33], [50, 7, 40], 7, 16, 4, 32),
    ("prefill_only", [129, 64], [300, 64], 20, 8, 2, 16),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
def test_cascade_small(ci):
    name, ql, own, P, hq, hkv, bs = CASES[ci]
    say(f"cascade {name}")
    b = _batch(500 + ci, ql, own, P, hq, hkv, bs)
    plan = _plan(b, P)
    assert plan.prefix_len == P * bs
    cache_t, out, lse = _run(b, plan)
    cache_ref, oref, lref = _oracle(b)
    assert np.array_equal(bits(cache_t), cache_ref)
    _check_rows(b, out, lse, oref, lref, range(b.num_seqs), name)


def test_cascade_key_range_cuts():
    """Different compute-unit counts cut the prefix into different key ranges
    (one range up to many, each a multiple of 64 keys, the last ragged)."""
    say("cascade key-range cuts")
    b = _batch(520, [1] * 6 + [40], [3, 500, 80, 1, 260, 9, 100], 137, 32, 8)
    cache_ref, oref, lref = _oracle(b)
    seen = set()
    for cus in (1, 16, 80, 256, 4096):
        plan = _plan(b, 137, cus)
        seen.add(plan.prefix_splits)
        _, out, lse = _run(b, plan)
        _check_rows(b, out, lse, oref, lref, range(b.num_seqs), f"{cus} CUs")
    assert len(seen) >= 3, seen


def test_cascade_without_prefix_is_the_mixed_path():
    """P = 0: the plan is a mixed-batch plan and the run is bit for bit
    pa_mixed_attention's."""
    say("cascade P = 0")
    b = _batch(530, [1, 1, 1, 60], [900, 3000, 20, 200], 0, 16, 4)
    plan = _plan(b, 0)
    assert plan.prefix_len == 0 and plan.workspace_bytes == plan.suffix.workspace_bytes
    _, out, lse = _run(b, plan)
    mp = pa.plan_mixed(b.query_start_loc, b.seq_lens, 16, 4, 128, 16, b.block_table.shape[1])
    cache_t = to_dev(b.cache)
    out2, lse2 = pa.mixed_attention(mp, to_dev(b.q), cache_t, to_dev(b.block_table),
                                    to_dev(b.query_start_loc), to_dev(b.seq_lens), b.scale,
                                    k=to_dev(b.k_new), v=to_dev(b.v_new),
                                    slot_mapping=to_dev(b.slot_mapping))
    torch.cuda.synchronize()
    assert np.array_equal(out, to_f64(out2))
    assert np.array_equal(lse, lse2.cpu().numpy().astype(np.float64))


def test_cascade_plan_serves_every_layer():
    say("cascade plan reused across layers")
    ql, own, P = [1, 1, 1, 50], [700, 20, 1500, 50], 64
    plan = _plan(_batch(540, ql, own, P, 32, 8), P)
    for layer in range(3):
        b = _batch(np.random.default_rng(600 + layer), ql, own, P, 32, 8)
        cache_t, out, lse = _run(b, plan)
        cache_ref, oref, lref = _oracle(b)
        assert np.array_equal(bits(cache_t), cache_ref)
        _check_rows(b, out, lse, oref, lref, range(b.num_seqs), f"layer {layer}")


def test_cascade_deterministic():
    say("cascade determinism")
    b = _batch(550, [1, 1, 1, 30], [300, 60, 2000, 31], 90, 16, 4)
    plan = _plan(b, 90)
    _, o1, l1 = _run(b, plan)
    _, o2, l2 = _run(b, plan)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.fixture(scope="module")
def shared():
    return W.cascade_batch()


def test_cascade_workload_full_size(shared):
    """64 decode requests sharing a 4096-token prefix, own U{512..4096}
    tokens, 32/8 heads: 16 sampled requests (longest and shortest among them)
    against the oracle, the cache bit-exact."""
    b = shared
    plan = _plan(b, 256)
    say(f"cascade full size: {plan}")
    cache_t, out, lse = _run(b, plan)
    assert np.all(np.isfinite(out))
    pick = np.random.default_rng(8).choice(64, size=14, replace=False)
    reqs = sorted(set([int(x) for x in pick] + [int(np.argmax(b.seq_lens)),
                                                int(np.argmin(b.seq_lens))]))
    cache_ref, oref, lref = _oracle(b, requests=reqs)
    _check_rows(b, out, lse, oref, lref, reqs, "cascade workload")
    assert np.array_equal(bits(cache_t), cache_ref)
