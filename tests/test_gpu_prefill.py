"""GPU parity of pa_prefill_varlen (write + varlen causal attention) against
the oracle: ragged chunk lengths and contexts that span several 128-row and
64-key tiles with ragged tails, every supported GQA group, causal and
unmasked, and sampled requests of the full chunked-prefill workload."""
import math

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _run(b: W.GqaBatch, causal=True, write=True):
    cache_t = to_dev(b.cache)
    out, lse = pa.prefill_varlen(
        to_dev(b.q), cache_t, to_dev(b.block_table), to_dev(b.query_start_loc),
        to_dev(b.seq_lens), b.max_query_len, b.max_seq_len, b.scale,
        k=to_dev(b.k_new) if write else None, v=to_dev(b.v_new) if write else None,
        slot_mapping=to_dev(b.slot_mapping) if write else None, causal=causal)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(b: W.GqaBatch, causal=True, requests=None):
    cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
    out, lse = O.paged_attention(b.q, cache, b.block_table, b.query_start_loc, b.seq_lens,
                                 b.scale, causal=causal, requests=requests)
    return cache, out, lse


CASES = [
    # name, q_lens, ctx_lens, Hq, Hkv, block_size
    ("ragged_g4", [1, 7, 64, 65, 130, 257], [0, 100, 0, 33, 511, 64], 8, 2, 16),
    ("long_chunk_g8", [300], [1000], 8, 1, 16),
    ("g1_block32", [129, 3], [31, 700], 2, 2, 32),
    ("g2_no_ctx", [200, 128], [0, 0], 4, 2, 16),
    ("g4_32_8", [90, 40, 260], [17, 256, 4], 32, 8, 16),
    # requests with no query rows (L_r = 0) between others
    ("empty_chunks_g4", [0, 70, 129, 0, 5], [40, 50, 100, 1, 300], 32, 8, 16),
    # page sizes that are multiples of 16 but not powers of two
    ("g4_block48_empty", [0, 70, 129, 33], [40, 50, 100, 17], 32, 8, 48),
    ("g8_block80", [200, 33], [90, 400], 16, 2, 80),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_prefill_small(ci, causal):
    name, ql, cl, hq, hkv, bs = CASES[ci]
    say(f"prefill {name} causal={causal}")
    seq = np.array(ql) + np.array(cl)
    b = W.make_gqa(200 + ci, ql, seq, hq, hkv, 128, bs, W.BF16, scale=1.1 / math.sqrt(128))
    cache_t, out, lse = _run(b, causal=causal)
    cache_ref, oref, lref = _oracle(b, causal=causal)
    assert np.array_equal(bits(cache_t), cache_ref)
    check_close(out, oref, f"{name} out")
    check_lse(lse, lref, f"{name} lse")


def test_prefill_len1_matches_decode():
    """A chunk of one query per request is a decode step."""
    say("prefill L=1 vs decode")
    b = W.make_gqa(7, [1, 1, 1], [1, 90, 1500], 16, 4, 128, 16, W.BF16)
    _, out_p, lse_p = _run(b)
    cache_t = to_dev(b.cache)
    out_d, lse_d = pa.decode(to_dev(b.q), cache_t, to_dev(b.block_table), to_dev(b.seq_lens),
                             b.max_seq_len, b.scale, k=to_dev(b.k_new), v=to_dev(b.v_new),
                             slot_mapping=to_dev(b.slot_mapping), num_splits=1)
    torch.cuda.synchronize()
    check_close(out_p, to_f64(out_d), "prefill vs decode", atol=1e-2, rtol=1e-2)
    check_lse(lse_p, lse_d.cpu().numpy().astype(np.float64), "prefill vs decode lse")


def test_prefill_two_chunks_equal_one_shot():
    """Chunk 2 of a prompt (after chunk 1 was written) gives the rows a
    one-shot prefill gives for the same positions."""
    say("prefill two chunks")
    S, c1 = 700, 300
    one = W.make_gqa(9, [S], [S], 8, 2, 128, 16, W.BF16)
    _, out_one, lse_one = _run(one)
    # chunk 1 then chunk 2 on one cache, same table and values
    cache_t = to_dev(one.cache)
    bt, qsl = to_dev(one.block_table), None
    for lo, hi in ((0, c1), (c1, S)):
        qsl = to_dev(np.array([0, hi - lo], dtype=np.int32))
        out, lse = pa.prefill_varlen(
            to_dev(one.q[lo:hi]), cache_t, bt, qsl, to_dev(np.array([hi], np.int32)), hi - lo, hi,
            one.scale, k=to_dev(one.k_new[lo:hi]), v=to_dev(one.v_new[lo:hi]),
            slot_mapping=to_dev(one.slot_mapping[lo:hi]))
    torch.cuda.synchronize()
    check_close(to_f64(out), out_one[c1:], "chunked vs one-shot", atol=1e-2, rtol=1e-2)
    check_lse(lse.cpu().numpy().astype(np.float64), lse_one[c1:], "chunked vs one-shot lse")


def test_prefill_deterministic_and_permutation_invariant():
    say("prefill determinism / block permutation")
    b = W.make_gqa(11, [150, 70], [350, 70], 8, 2, 128, 16, W.BF16)
    _, o1, l1 = _run(b)
    _, o2, l2 = _run(b)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(3).permutation(b.num_blocks)
    cache2 = np.empty_like(b.cache)
    cache2[perm] = b.cache
    bb = W.GqaBatch(**{**b.__dict__, "cache": cache2,
                       "block_table": perm[b.block_table].astype(np.int32),
                       "slot_mapping": (perm[b.slot_mapping // 16] * 16 + b.slot_mapping % 16)})
    _, o3, l3 = _run(bb)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


@pytest.fixture(scope="module")
def chunked():
    return W.chunked_prefill()


def test_chunked_prefill_full_size(chunked):
    """16 requests, chunks U{64..2048} over contexts U{0..4096}, 32/8 heads."""
    b = chunked
    say(f"prefill full size T={b.num_tokens}")
    cache_t, out, lse = _run(b)
    assert np.all(np.isfinite(out))
    reqs = [int(np.argmax(b.q_lens)), int(np.argmin(b.q_lens)),
            int(np.argmax(b.seq_lens - b.q_lens)), int(np.argmin(b.seq_lens - b.q_lens))]
    cache_ref, oref, lref = _oracle(b, requests=sorted(set(reqs)))
    for r in sorted(set(reqs)):
        a0, a1 = b.query_start_loc[r], b.query_start_loc[r + 1]
        check_close(out[a0:a1], oref[a0:a1], f"request {r}")
        check_lse(lse[a0:a1], lref[a0:a1], f"request {r}")
    assert np.array_equal(bits(cache_t), cache_ref)


def test_prefill_scale_zero_is_uniform_attention():
    """scale = 0: every visible key weighs the same (masked keys still none)."""
    say("prefill scale 0")
    b = W.make_gqa(13, [100, 3], [300, 3], 8, 2, 128, 16, W.BF16, scale=0.0)
    _, out, lse = _run(b)
    _, oref, lref = _oracle(b)
    check_close(out, oref, "scale 0 out")
    check_lse(lse, lref, "scale 0 lse")


@pytest.mark.parametrize("ql,ctx", [(64, 65472), (64, 65808)], ids=["at_table_limit", "past_table"])
def test_prefill_long_context_table_limit(ql, ctx):
    """A request whose keys fill the bf16 prefill's 16-key-group address
    table exactly (65536 keys: the ping-pong kernel), and one past it
    (65872 keys: the launcher takes the 4-wave kernel instead); every row
    against the oracle."""
    say(f"prefill long context {ql} rows over {ctx + ql} keys")
    b = W.make_gqa(290, [ql], np.array([ql + ctx]), 4, 1, 128, 16, W.BF16,
                   scale=1.0 / math.sqrt(128))
    cache_t, out, lse = _run(b)
    _, oref, lref = _oracle(b)
    check_close(out, oref, f"long context {ctx + ql} out")
    check_lse(lse, lref, f"long context {ctx + ql} lse")
