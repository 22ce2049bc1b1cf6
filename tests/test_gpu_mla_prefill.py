"""GPU parity of MLA prefill in the multi-head form (pa_mla_prefill: latent
write, projection of every key by kv_b_proj, causal attention with 192-wide
keys and 128-wide values) against the oracle: ragged chunks over contexts
that span several 128-row query tiles and 64-key tiles with ragged tails,
one-query and empty requests, head counts 1 to 16, block sizes 16 and 64,
strided queries, a 70000-key context (the work list's coarsened sort), and
sampled requests of the full workload."""
import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _run(b, q_pad=0, write=True):
    cache_t = to_dev(b.cache)
    q = to_dev(b.q)
    if q_pad:   # the queries as a view of wider rows (q_stride_h = 192 + q_pad)
        wide = torch.zeros((b.num_tokens, b.num_heads, 192 + q_pad), dtype=torch.bfloat16,
                           device=q.device)
        wide[:, :, :192] = q
        q = wide[:, :, :192]
    out, lse = pa.mla_prefill(q, cache_t, to_dev(b.block_table), to_dev(b.query_start_loc),
                              to_dev(b.seq_lens), to_dev(b.w_kv_b), b.max_query_len, b.total_keys,
                              b.scale, kv_c=to_dev(b.kv_c_new) if write else None,
                              k_pe=to_dev(b.k_pe_new) if write else None,
                              slot_mapping=to_dev(b.slot_mapping) if write else None)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(b, requests=None):
    cache = O.cache_write_mla(b.cache, b.kv_c_new, b.k_pe_new, b.slot_mapping)
    w = b.w_kv_b.reshape(b.num_heads, 256, 512)
    out, lse = O.mla_prefill(b.q, cache, w, b.block_table, b.query_start_loc, b.seq_lens,
                             b.scale, qk_nope=128, requests=requests)
    return cache, out, lse


def _check(b, out, lse, oref, lref, requests, what):
    for r in requests:
        a0, a1 = b.query_start_loc[r], b.query_start_loc[r + 1]
        check_close(out[a0:a1], oref[a0:a1], f"{what} request {r} out")
        check_lse(lse[a0:a1], lref[a0:a1], f"{what} request {r} lse")


CASES = [
    # name, q_lens, context lens, heads, block size
    ("ragged_h4", [1, 7, 130, 64, 0, 257], [0, 100, 33, 511, 20, 64], 4, 64),
    ("long_chunk_h1", [300], [700], 1, 64),
    ("block16_h2", [129, 3, 1], [31, 200, 5], 2, 16),
    ("no_context_h16", [200, 128], [0, 0], 16, 64),
    ("odd_heads_h5", [90, 1, 45], [17, 900, 64], 5, 64),
    # a request with no keys at all and one with keys but no queries
    ("empty_requests_h8", [5, 0, 0, 9], [0, 0, 3, 0], 8, 16),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
def test_mla_prefill_small(ci):
    name, ql, cl, H, bs = CASES[ci]
    say(f"mla prefill {name}")
    b = W.make_mla_prefill(800 + ci, ql, np.array(ql) + np.array(cl), H, bs)
    cache_t, out, lse = _run(b)
    cache_ref, oref, lref = _oracle(b)
    assert np.array_equal(bits(cache_t), cache_ref)
    _check(b, out, lse, oref, lref, range(b.num_seqs), name)


def test_mla_prefill_strided_queries():
    say("mla prefill strided q")
    b = W.make_mla_prefill(810, [70, 5], [300, 5], 3, 64)
    _, out, lse = _run(b, q_pad=64)
    _, oref, lref = _oracle(b)
    _check(b, out, lse, oref, lref, range(b.num_seqs), "strided")


def test_mla_prefill_one_query_matches_latent_decode():
    """A chunk of one query per request is a decode step: the multi-head
    form equals the latent (absorbed) form run by pa_mla_decode with the
    query projected by W_k and its latent output projected by W_v, up to the
    bf16 roundings of the two paths."""
    say("mla prefill vs latent decode")
    H = 16
    b = W.make_mla_prefill(820, [1, 1, 1], [1, 300, 2000], H, 64)
    _, out, lse = _run(b)
    w = O.to_f64(b.w_kv_b.reshape(H, 256, 512))
    q = O.to_f64(b.q)
    q_lat = np.einsum("bhd,hdr->bhr", q[:, :, :128], w[:, :128, :])
    q_lat_t = torch.from_numpy(q_lat.astype(np.float32)).to(torch.bfloat16).cuda()
    cache_t = to_dev(O.cache_write_mla(b.cache, b.kv_c_new, b.k_pe_new, b.slot_mapping))
    lat, lse_d, _, _ = pa.mla_decode_balanced(q_lat_t, to_dev(b.q)[:, :, 128:].contiguous(), cache_t,
                                              to_dev(b.block_table), to_dev(b.seq_lens), b.scale)
    torch.cuda.synchronize()
    o_dec = np.einsum("bhr,hvr->bhv", to_f64(lat), w[:, 128:, :])
    # both paths round intermediates to bf16 (projected keys / the latent
    # query and output): compare against each other at twice the tolerance
    check_close(out, o_dec, "prefill vs decode", atol=2e-2, rtol=2e-2)
    check_lse(lse, lse_d.cpu().numpy().astype(np.float64), "prefill vs decode lse", tol=2e-2)


def test_mla_prefill_long_context_coarse_schedule():
    """A 70000-key context: the work list's sort key (key tiles of a request's
    last q tile) exceeds the 1024 buckets, so the schedule coarsens it; the
    result must not change."""
    say("mla prefill 70000-key context")
    b = W.make_mla_prefill(840, [64, 1], [70000, 5], 1, 64)
    _, out, lse = _run(b)
    _, oref, lref = _oracle(b)
    _check(b, out, lse, oref, lref, range(b.num_seqs), "long context")


def test_mla_prefill_deterministic():
    say("mla prefill determinism")
    b = W.make_mla_prefill(830, [100, 40], [400, 40], 4, 64)
    _, o1, l1 = _run(b)
    _, o2, l2 = _run(b)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.fixture(scope="module")
def full():
    return W.mla_prefill_batch()


def test_mla_prefill_workload_full_size(full):
    """16 requests, chunks U{64..2048} over contexts U{0..4096}, 16 heads:
    the shortest and the longest chunk against the oracle, cache bit-exact."""
    b = full
    say(f"mla prefill full size T={b.num_tokens} keys={b.total_keys}")
    cache_t, out, lse = _run(b)
    assert np.all(np.isfinite(out))
    reqs = sorted({int(np.argmax(b.q_lens)), int(np.argmin(b.q_lens))})
    cache_ref, oref, lref = _oracle(b, requests=reqs)
    _check(b, out, lse, oref, lref, reqs, "workload")
    assert np.array_equal(bits(cache_t), cache_ref)
