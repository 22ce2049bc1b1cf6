"""GPU parity of the FP8 (E4M3) KV cache: the quantising cache write is
bit-exact against the oracle's (GQA and MLA layouts, saturation, the
unaligned path), and decode over an FP8 cache matches the oracle's attention
over the dequantised cache for every supported GQA group and head count,
ragged lengths, block sizes 16 and 32, and sampled requests of the full
FP8 decode workload; MLA decode over an FP8 latent cache likewise.  With
power-of-two scales the dequantised values are bf16 values, and the FP8
kernels equal the bf16 kernels over them bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _host(t):
    return t.cpu().numpy()


def test_fp8_write_gqa_bit_exact():
    say("fp8 write gqa")
    rng = np.random.default_rng(700)
    b = W.make_gqa(rng, [1, 5, 9, 1], [40, 5, 300, 17], 16, 4, 128, 16, W.FP8)
    slots = b.slot_mapping.copy()
    slots[2] = -1                               # not written
    for ks, vs in ((0.25, 0.5), (0.037, 1.7), (0.001, 0.0005)):   # the last saturates
        cache_t = _u8(b.cache)
        pa.cache_write_fp8(cache_t, to_dev(b.k_new), to_dev(b.v_new), to_dev(slots), ks, vs)
        torch.cuda.synchronize()
        ref = O.cache_write_kv_fp8(b.cache, b.k_new, b.v_new, slots, ks, vs)
        got = _host(cache_t)
        assert np.array_equal(got, ref), (ks, vs, int((got != ref).sum()))
    assert (ref == 0x7E).any() or (ref == 0xFE).any()   # saturation exercised


def test_fp8_write_unaligned_rows():
    """k / v starting one element past a 16-byte boundary take the
    one-element path and store the same bytes."""
    say("fp8 write unaligned")
    b = W.make_gqa(701, [3, 2], [3, 10], 8, 2, 128, 16, W.FP8)
    T = b.num_tokens
    kb = torch.empty(T * 2 * 128 + 1, dtype=torch.bfloat16, device="cuda:0")
    vb = torch.empty_like(kb)
    k_t = kb[1:].view(T, 2, 128)
    v_t = vb[1:].view(T, 2, 128)
    k_t.copy_(to_dev(b.k_new))
    v_t.copy_(to_dev(b.v_new))
    cache_t = _u8(b.cache)
    pa.cache_write_fp8(cache_t, k_t, v_t, to_dev(b.slot_mapping), 0.3, 0.07)
    torch.cuda.synchronize()
    ref = O.cache_write_kv_fp8(b.cache, b.k_new, b.v_new, b.slot_mapping, 0.3, 0.07)
    assert np.array_equal(_host(cache_t), ref)


def test_fp8_write_mla_bit_exact():
    say("fp8 write mla")
    rng = np.random.default_rng(702)
    nb, bs, T = 9, 64, 7
    cache = np.full((nb, bs, 576), 0x7F, np.uint8)
    kv_c = W._normal(rng, (T, 512), W.BF16)
    k_pe = W._normal(rng, (T, 64), W.BF16)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    cache_t = _u8(cache)
    pa.cache_write_fp8(cache_t, to_dev(kv_c), to_dev(k_pe), to_dev(slots), 0.05,
                       layout=pa.PA_LAYOUT_MLA)
    torch.cuda.synchronize()
    ref = O.cache_write_mla_fp8(cache, kv_c, k_pe, slots, 0.05)
    assert np.array_equal(_host(cache_t), ref)


def _run(b, write=True, num_ranges=0):
    cache_t = _u8(b.cache)
    out, lse = pa.decode_fp8(to_dev(b.q), cache_t, to_dev(b.block_table), to_dev(b.seq_lens),
                             b.scale, b.k_scale, b.v_scale,
                             k=to_dev(b.k_new) if write else None,
                             v=to_dev(b.v_new) if write else None,
                             slot_mapping=to_dev(b.slot_mapping) if write else None,
                             num_ranges=num_ranges)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(b, requests=None):
    cache = O.cache_write_kv_fp8(b.cache, b.k_new, b.v_new, b.slot_mapping, b.k_scale, b.v_scale)
    deq = O.dequant_kv_cache(cache, b.k_scale, b.v_scale)
    out, lse = O.paged_decode(b.q, deq, b.block_table, b.seq_lens, b.scale, requests=requests)
    return cache, out, lse


CASES = [
    # name, seq_lens, Hq, Hkv, block size, k_scale, v_scale
    ("g4_8kv", [1, 31, 32, 33, 700, 2049, 5000, 64], 32, 8, 16, 0.3, 0.07),
    ("g8_1kv", [1, 2, 900, 129, 4097], 8, 1, 16, 0.25, 0.5),
    ("g1_4kv", [17, 3000, 1, 250], 4, 4, 32, 1.3, 0.011),
    ("g2_2kv", [600, 5, 1111], 4, 2, 16, 0.02, 2.0),
    ("g4_16kv", [1, 100, 3333, 64, 65], 64, 16, 16, 0.125, 0.75),
    # page sizes that are multiples of 16 but not powers of two
    ("g4_8kv_bs48", [47, 49, 700, 2000], 32, 8, 48, 0.3, 0.07),
    ("g8_1kv_bs80", [79, 81, 1500], 8, 1, 80, 0.25, 0.5),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
def test_fp8_decode_small(ci):
    name, sl, hq, hkv, bs, ks, vs = CASES[ci]
    say(f"fp8 decode {name}")
    b = W.make_gqa(710 + ci, np.ones(len(sl), np.int64), sl, hq, hkv, 128, bs, W.FP8,
                   scale=1.0 / math.sqrt(128), k_scale=ks, v_scale=vs)
    cache_t, out, lse = _run(b)
    cache_ref, oref, lref = _oracle(b)
    assert np.array_equal(_host(cache_t), cache_ref)
    check_close(out, oref, f"{name} out")
    check_lse(lse, lref, f"{name} lse")


def test_fp8_decode_range_counts():
    """Other range counts cut the chunk list elsewhere; every cut agrees with
    the oracle."""
    say("fp8 decode range counts")
    b = W.make_gqa(720, np.ones(6, np.int64), [1, 800, 64, 3000, 33, 1500], 16, 4, 128, 16,
                   W.FP8, k_scale=0.4, v_scale=0.09)
    _, oref, lref = _oracle(b)
    for nr in (1, 3, 64, 1000):
        _, out, lse = _run(b, num_ranges=nr)
        check_close(out, oref, f"{nr} ranges out")
        check_lse(lse, lref, f"{nr} ranges lse")


def test_fp8_decode_equals_bf16_decode_on_dequantised_cache():
    """Power-of-two scales: code * scale is a bf16 value, and the FP8 kernel
    (scores on the codes, scales folded into the softmax and the output)
    gives the bf16 kernel's result on the dequantised cache bit for bit."""
    say("fp8 vs bf16 decode")
    b = W.make_gqa(730, np.ones(5, np.int64), [3, 1000, 77, 4000, 600], 32, 8, 128, 16, W.FP8,
                   k_scale=0.25, v_scale=2.0)
    cache_t, out8, lse8 = _run(b)
    deq = O.fp8_e4m3_to_f64(_host(cache_t))
    deq[:, 0] *= b.k_scale
    deq[:, 1] *= b.v_scale
    deq = np.where(np.isnan(deq), 0.0, deq)
    bf = W.f32_to_bf16_bits(deq.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(bf), deq.astype(np.float32))   # exact
    out16, lse16, _, _ = pa.decode_balanced(to_dev(b.q), to_dev(bf), to_dev(b.block_table),
                                            to_dev(b.seq_lens), b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(out8, to_f64(out16))
    assert np.array_equal(lse8, lse16.cpu().numpy().astype(np.float64))


@pytest.fixture(scope="module")
def fp8_batch():
    return W.llama_decode_fp8()


def test_fp8_decode_workload_full_size(fp8_batch):
    """64 requests U{512..8192} over an FP8 cache, 32/8 heads: 16 sampled
    requests against the oracle, the written cache bit-exact."""
    b = fp8_batch
    say(f"fp8 decode full size, {int(b.seq_lens.sum())} keys")
    cache_t, out, lse = _run(b)
    assert np.all(np.isfinite(out))
    reqs = sorted(set([int(x) for x in np.random.default_rng(9).choice(64, 14, replace=False)] +
                      [int(np.argmax(b.seq_lens)), int(np.argmin(b.seq_lens))]))
    cache_ref, oref, lref = _oracle(b, requests=reqs)
    for r in reqs:
        check_close(out[r], oref[r], f"request {r} out")
        check_lse(lse[r], lref[r], f"request {r} lse")
    assert np.array_equal(_host(cache_t), cache_ref)


# ------------------------------------------------------------------ MLA
def _run_mla(b, write=True, num_ranges=0):
    cache_t = _u8(b.cache)
    out, lse = pa.mla_decode_fp8(to_dev(b.q_nope), to_dev(b.q_pe), cache_t, to_dev(b.block_table),
                                 to_dev(b.seq_lens), b.scale, b.kv_scale,
                                 kv_c=to_dev(b.kv_c_new) if write else None,
                                 k_pe=to_dev(b.k_pe_new) if write else None,
                                 slot_mapping=to_dev(b.slot_mapping) if write else None,
                                 num_ranges=num_ranges)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle_mla(b, requests=None):
    cache = O.cache_write_mla_fp8(b.cache, b.kv_c_new, b.k_pe_new, b.slot_mapping, b.kv_scale)
    deq = O.dequant_mla_cache(cache, b.kv_scale)
    out, lse = O.mla_decode(b.q_nope, b.q_pe, deq, b.block_table, b.seq_lens, b.scale,
                            requests=requests)
    return cache, out, lse


MLA_CASES = [
    # name, seq_lens, heads, block size, kv_scale
    ("h128_bs64", [1, 31, 32, 33, 700, 2049, 64], 128, 64, 0.3),
    ("h16_bs16", [5, 1, 129, 1000], 16, 16, 0.07),
    ("h64_bs32_long", [3000, 2, 95], 64, 32, 1.5),
    ("h112_bs64", [40, 513], 112, 64, 0.25),
    ("h128_bs48", [47, 49, 1000], 128, 48, 0.3),
    ("h32_bs80", [79, 81, 1700], 32, 80, 0.2),
]


@pytest.mark.parametrize("ci", range(len(MLA_CASES)), ids=[c[0] for c in MLA_CASES])
def test_fp8_mla_small(ci):
    name, sl, H, bs, sc = MLA_CASES[ci]
    say(f"fp8 mla {name}")
    b = W.make_mla(740 + ci, sl, H, 512, 64, bs, cache_dtype=W.FP8, kv_scale=sc)
    cache_t, out, lse = _run_mla(b)
    cache_ref, oref, lref = _oracle_mla(b)
    assert np.array_equal(_host(cache_t), cache_ref)
    check_close(out, oref, f"{name} out")
    check_lse(lse, lref, f"{name} lse")


def test_fp8_mla_range_counts():
    say("fp8 mla range counts")
    b = W.make_mla(750, [1, 900, 64, 3000, 33], 32, 512, 64, 64, cache_dtype=W.FP8, kv_scale=0.2)
    _, oref, lref = _oracle_mla(b)
    for nr in (1, 5, 77, 700):
        _, out, lse = _run_mla(b, num_ranges=nr)
        check_close(out, oref, f"{nr} ranges out")
        check_lse(lse, lref, f"{nr} ranges lse")


def test_fp8_mla_equals_bf16_mla_on_dequantised_cache():
    """Power-of-two scale: the FP8 MLA kernel (tiles widened in LDS, the scale
    folded into the softmax and the output) gives the bf16 MLA kernel's
    result over the dequantised cache bit for bit."""
    say("fp8 mla vs bf16 mla")
    b = W.make_mla(760, [3, 1000, 77, 4000, 600, 64], 128, 512, 64, 64, cache_dtype=W.FP8,
                   kv_scale=0.5)
    cache_t, out8, lse8 = _run_mla(b)
    deq = O.fp8_e4m3_to_f64(_host(cache_t)) * b.kv_scale
    deq = np.where(np.isnan(deq), 0.0, deq)
    bf = W.f32_to_bf16_bits(deq.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(bf), deq.astype(np.float32))
    out16, lse16, _, _ = pa.mla_decode_balanced(to_dev(b.q_nope), to_dev(b.q_pe), to_dev(bf),
                                                to_dev(b.block_table), to_dev(b.seq_lens), b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(out8, to_f64(out16))
    assert np.array_equal(lse8, lse16.cpu().numpy().astype(np.float64))


@pytest.fixture(scope="module")
def fp8_mla_batch():
    return W.mla_decode_fp8_batch()


def test_fp8_mla_workload_full_size(fp8_mla_batch):
    """128 requests U{1024..8192}, 128 heads, FP8 latent cache: 12 sampled
    requests against the oracle, the written cache bit-exact."""
    b = fp8_mla_batch
    say(f"fp8 mla full size, {int(b.seq_lens.sum())} keys")
    cache_t, out, lse = _run_mla(b)
    assert np.all(np.isfinite(out))
    reqs = sorted(set([int(x) for x in np.random.default_rng(10).choice(128, 10, replace=False)] +
                      [int(np.argmax(b.seq_lens)), int(np.argmin(b.seq_lens))]))
    cache_ref, oref, lref = _oracle_mla(b, requests=reqs)
    for r in reqs:
        check_close(out[r], oref[r], f"request {r} out")
        check_lse(lse[r], lref[r], f"request {r} lse")
    assert np.array_equal(_host(cache_t), cache_ref)


# -------------------------------------------------------------- prefill
def _run_prefill(b, causal=True):
    cache_t = _u8(b.cache)
    out, lse = pa.prefill_varlen_fp8(to_dev(b.q), cache_t, to_dev(b.block_table),
                                     to_dev(b.query_start_loc), to_dev(b.seq_lens), b.max_query_len,
                                     b.max_seq_len, b.scale, b.k_scale, b.v_scale,
                                     k=to_dev(b.k_new), v=to_dev(b.v_new),
                                     slot_mapping=to_dev(b.slot_mapping), causal=causal)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle_prefill(b, causal=True, requests=None):
    cache = O.cache_write_kv_fp8(b.cache, b.k_new, b.v_new, b.slot_mapping, b.k_scale, b.v_scale)
    deq = O.dequant_kv_cache(cache, b.k_scale, b.v_scale)
    out, lse = O.paged_attention(b.q, deq, b.block_table, b.query_start_loc, b.seq_lens, b.scale,
                                 causal=causal, requests=requests)
    return cache, out, lse


PREFILL_CASES = [
    # name, q_lens, context lens, Hq, Hkv, block size, k_scale, v_scale
    ("ragged_g4", [1, 7, 64, 65, 130, 257], [0, 100, 0, 33, 511, 64], 8, 2, 16, 0.3, 0.07),
    ("long_chunk_g8", [300], [1000], 8, 1, 16, 0.25, 0.5),
    ("g1_block32", [129, 3], [31, 700], 2, 2, 32, 1.3, 0.011),
    ("g4_32_8", [90, 40, 260], [17, 256, 4], 32, 8, 16, 0.02, 2.0),
    ("g4_bs48_empty", [0, 70, 129], [40, 50, 100], 32, 8, 48, 0.3, 0.07),
    ("g8_bs80", [200, 33], [90, 400], 16, 2, 80, 0.25, 0.5),
]


@pytest.mark.parametrize("ci", range(len(PREFILL_CASES)), ids=[c[0] for c in PREFILL_CASES])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_fp8_prefill_small(ci, causal):
    name, ql, cl, hq, hkv, bs, ks, vs = PREFILL_CASES[ci]
    say(f"fp8 prefill {name} causal={causal}")
    b = W.make_gqa(770 + ci, ql, np.array(ql) + np.array(cl), hq, hkv, 128, bs, W.FP8,
                   scale=1.0 / math.sqrt(128), k_scale=ks, v_scale=vs)
    cache_t, out, lse = _run_prefill(b, causal)
    cache_ref, oref, lref = _oracle_prefill(b, causal)
    assert np.array_equal(_host(cache_t), cache_ref)
    check_close(out, oref, f"{name} out")
    check_lse(lse, lref, f"{name} lse")


def test_fp8_prefill_equals_bf16_prefill_on_dequantised_cache():
    """Power-of-two scales: the FP8 prefill equals the bf16 prefill over the
    dequantised cache bit for bit (same tiles, same arithmetic after the
    exact widening)."""
    say("fp8 prefill vs bf16 prefill")
    b = W.make_gqa(780, [150, 1, 70], [400, 90, 70], 16, 4, 128, 16, W.FP8, k_scale=0.125,
                   v_scale=4.0)
    cache_t, out8, lse8 = _run_prefill(b)
    deq = O.fp8_e4m3_to_f64(_host(cache_t))
    deq[:, 0] *= b.k_scale
    deq[:, 1] *= b.v_scale
    deq = np.where(np.isnan(deq), 0.0, deq)
    bf = W.f32_to_bf16_bits(deq.astype(np.float32))
    out16, lse16 = pa.prefill_varlen(to_dev(b.q), to_dev(bf), to_dev(b.block_table),
                                     to_dev(b.query_start_loc), to_dev(b.seq_lens), b.max_query_len,
                                     b.max_seq_len, b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(out8, to_f64(out16))
    assert np.array_equal(lse8, lse16.cpu().numpy().astype(np.float64))


def test_fp8_prefill_workload_full_size():
    """The chunked-prefill shape over an FP8 cache: 16 requests, chunks
    U{64..2048} over contexts U{0..4096}, 32/8 heads; the longest and the
    shortest chunk against the oracle."""
    b = W.chunked_prefill_fp8()
    say(f"fp8 prefill full size T={b.num_tokens}")
    cache_t, out, lse = _run_prefill(b)
    assert np.all(np.isfinite(out))
    reqs = sorted({int(np.argmax(b.q_lens)), int(np.argmin(b.q_lens))})
    cache_ref, oref, lref = _oracle_prefill(b, requests=reqs)
    for r in reqs:
        a0, a1 = b.query_start_loc[r], b.query_start_loc[r + 1]
        check_close(out[a0:a1], oref[a0:a1], f"request {r} out")
        check_lse(lse[a0:a1], lref[a0:a1], f"request {r} lse")
    assert np.array_equal(_host(cache_t), cache_ref)
