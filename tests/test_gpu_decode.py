"""GPU parity of pa_cache_write, pa_decode and pa_lse_merge against the oracle.

Element by element on seeded inputs at sizes the oracle finishes in seconds
(several 16-token groups, ragged tails, every split count), and on sampled
requests of the full-size workloads.  Cache writes and integer work are
bit-exact; outputs are within |gpu - oracle| <= 1e-2 + 1e-2 |oracle|; LSE
within 1e-3.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W
from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _run_decode(b: W.GqaBatch, num_splits=0, write=True, cache=None):
    """Upload a batch, run pa_decode (with the fused write), return host arrays."""
    cache_t = to_dev(b.cache) if cache is None else cache
    q = to_dev(b.q)
    out, lse = pa.decode(q, cache_t, to_dev(b.block_table), to_dev(b.seq_lens), b.max_seq_len,
                         b.scale, k=to_dev(b.k_new) if write else None,
                         v=to_dev(b.v_new) if write else None,
                         slot_mapping=to_dev(b.slot_mapping) if write else None,
                         num_splits=num_splits)
    torch.cuda.synchronize()
    return cache_t, to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle_decode(b: W.GqaBatch, requests=None):
    cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
    out, lse = O.paged_decode(b.q, cache, b.block_table, b.seq_lens, b.scale, requests=requests)
    return cache, out, lse


# ----------------------------------------------------------------- writes
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_cache_write_bit_exact(dtype):
    say(f"cache_write gqa {dtype}")
    rng = np.random.default_rng(31)
    nb, bs, H, D, T = 37, 32, 4, 128, 50
    store = np.uint16 if dtype == W.BF16 else np.float32
    cache = rng.integers(0, 2 ** 16, size=(nb, 2, bs, H, D)).astype(np.uint16)
    if dtype == W.F32:
        cache = rng.standard_normal((nb, 2, bs, H, D)).astype(np.float32)
    k = (rng.integers(0, 2 ** 16, size=(T, H, D)).astype(np.uint16) if dtype == W.BF16
         else rng.standard_normal((T, H, D)).astype(np.float32))
    v = (rng.integers(0, 2 ** 16, size=(T, H, D)).astype(np.uint16) if dtype == W.BF16
         else rng.standard_normal((T, H, D)).astype(np.float32))
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[[3, 17]] = -1
    ref = O.cache_write_kv(cache, k, v, slots)
    ct = to_dev(cache)
    pa.cache_write(ct, to_dev(k), to_dev(v), to_dev(slots))
    torch.cuda.synchronize()
    got = bits(ct)
    assert got.dtype == store
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


def test_cache_write_mla_bit_exact():
    say("cache_write mla")
    rng = np.random.default_rng(32)
    nb, bs, T = 11, 64, 40
    cache = rng.integers(0, 2 ** 16, size=(nb, bs, 576)).astype(np.uint16)
    kvc = rng.integers(0, 2 ** 16, size=(T, 512)).astype(np.uint16)
    kpe = rng.integers(0, 2 ** 16, size=(T, 64)).astype(np.uint16)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[0] = -5
    ref = O.cache_write_mla(cache, kvc, kpe, slots)
    ct = to_dev(cache)
    pa.cache_write(ct, to_dev(kvc), to_dev(kpe), to_dev(slots), layout=pa.PA_LAYOUT_MLA)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ct), ref)


# ------------------------------------------------------------ small decode
def _small(seed, seq, hq, hkv, dtype, bs=16, scale=None):
    return W.make_gqa(seed, np.ones(len(seq), dtype=np.int64), seq, hq, hkv, 128, bs, dtype,
                      scale=scale)


CASES = [
    # (name, seq_lens, Hq, Hkv, block_size, dtype)
    ("ragged_g4_bf16", [1, 15, 16, 17, 33, 100, 257, 700], 32, 8, 16, W.BF16),
    ("g8_bf16", [5, 64, 1000, 2049], 64, 8, 16, W.BF16),
    ("g1_bf16", [3, 40, 511, 513], 8, 8, 16, W.BF16),
    ("g2_bf16_block32", [31, 32, 33, 900], 4, 2, 32, W.BF16),
    ("g2_hkv6_bf16", [300, 1200, 7], 12, 6, 16, W.BF16),   # automatic schedule: splits
    ("g4_fp32", [2, 128, 1025], 8, 2, 16, W.F32),
    ("g8_fp32_block64", [70, 640], 16, 2, 64, W.F32),
    # page sizes that are multiples of 16 but not powers of two
    ("g4_bf16_block48", [47, 48, 49, 700, 1500], 32, 8, 48, W.BF16),
    ("g8_bf16_block80", [79, 81, 2000], 64, 8, 80, W.BF16),
    ("g4_fp32_block48", [5, 95, 1000], 8, 2, 48, W.F32),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 64])
def test_decode_small(ci, splits):
    name, seq, hq, hkv, bs, dtype = CASES[ci]
    say(f"decode {name} splits={splits}")
    b = _small(100 + ci, seq, hq, hkv, dtype, bs=bs, scale=0.9 / math.sqrt(128))
    cache_t, out, lse = _run_decode(b, num_splits=splits)
    cache_ref, oref, lref = _oracle_decode(b)
    assert np.array_equal(bits(cache_t).view(np.uint8), cache_ref.view(np.uint8))
    check_close(out, oref, f"{name} out")
    check_lse(lse, lref, f"{name} lse")


@pytest.mark.parametrize("hkv", [8, 16])
def test_decode_writes_every_new_token(hkv):
    """The automatic (balanced) bf16 decode writes the step's new tokens
    itself: every request's row lands in its slot, also for a request whose
    seq_len is 0 (no key to attend, but a slot), and a negative slot is
    skipped; the cache after the call is the oracle's write bit for bit."""
    say(f"decode fused write hkv={hkv}")
    b = _small(119 + hkv, [300, 1, 900, 1, 17, 64], 4 * hkv, hkv, W.BF16)
    seq = b.seq_lens.copy()
    seq[[1, 3]] = 0
    b = dataclasses.replace(b, seq_lens=seq)
    b.slot_mapping[3] = -1   # a request with no key and no slot: nothing written
    cache_t, out, lse = _run_decode(b, num_splits=0)
    cache_ref, oref, lref = _oracle_decode(b)
    assert np.array_equal(bits(cache_t).view(np.uint8), cache_ref.view(np.uint8))
    assert np.all(out[[1, 3]] == 0) and np.all(np.isneginf(lse[[1, 3]]))
    check_close(out, oref, "fused write out")
    check_lse(lse, lref, "fused write lse")


def test_decode_tiny_workload():
    """3 requests (128, 1024, 4096 keys), fp32, 400-block pool, 8 splits."""
    b = W.tiny_decode()
    for splits in (0, 1, 8, 16):
        say(f"decode tiny_fp32 splits={splits}")
        cache_t, out, lse = _run_decode(b, num_splits=splits)
        _, oref, lref = _oracle_decode(b)
        check_close(out, oref, "tiny out")
        check_lse(lse, lref, "tiny lse")
        # fp32 end to end: much tighter than the bf16 bound
        assert np.max(np.abs(out - oref)) < 1e-4


def test_decode_without_write():
    say("decode no-write")
    b = _small(5, [17, 300], 8, 2, W.BF16)
    cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
    bb = W.GqaBatch(**{**b.__dict__, "cache": cache})
    _, out, lse = _run_decode(bb, num_splits=2, write=False)
    oref, lref = O.paged_decode(b.q, cache, b.block_table, b.seq_lens, b.scale)
    check_close(out, oref, "out")
    check_lse(lse, lref, "lse")


def test_decode_deterministic_and_permutation_invariant():
    """Same inputs -> same bits; moving physical blocks -> same bits."""
    say("decode determinism / block permutation")
    b = _small(77, [300, 1, 1500, 16], 32, 8, W.BF16)
    _, o1, l1 = _run_decode(b, num_splits=3)
    _, o2, l2 = _run_decode(b, num_splits=3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    rng = np.random.default_rng(5)
    perm = rng.permutation(b.num_blocks)
    cache2 = np.empty_like(b.cache)
    cache2[perm] = b.cache
    table2 = perm[b.block_table].astype(np.int32)
    slots2 = perm[b.slot_mapping // b.block_size] * b.block_size + b.slot_mapping % b.block_size
    b2 = W.GqaBatch(**{**b.__dict__, "cache": cache2, "block_table": table2,
                       "slot_mapping": slots2.astype(np.int64)})
    _, o3, l3 = _run_decode(b2, num_splits=3)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_split_counts_agree():
    """Every split count is within tolerance of the oracle and of the others."""
    say("decode split sweep")
    b = _small(8, [4000, 2500, 123], 32, 8, W.BF16)
    _, oref, lref = _oracle_decode(b)
    outs = []
    for s in (1, 2, 5, 8, 16, 250):
        _, o, l = _run_decode(b, num_splits=s)
        check_close(o, oref, f"splits={s}")
        check_lse(l, lref, f"splits={s}")
        outs.append(o)
    for o in outs[1:]:
        check_close(o, outs[0], "split vs unsplit", atol=2e-2, rtol=2e-2)


# ----------------------------------------------------------------- merge
@pytest.mark.parametrize("S,Dv,dtype", [(1, 128, torch.float32), (5, 128, torch.bfloat16),
                                        (300, 512, torch.bfloat16), (3, 1000, torch.float32)])
def test_lse_merge(S, Dv, dtype):
    say(f"lse_merge S={S} Dv={Dv}")
    rng = np.random.default_rng(S + Dv)
    R, H = 3, 5
    part = rng.standard_normal((R, H, S, Dv + 1)).astype(np.float32)
    part[..., Dv] *= 4
    part[0, 0, :, Dv] = -np.inf                          # all splits empty
    if S > 1:
        part[1, 2, 0, Dv] = -np.inf                      # one empty split
        part[1, 2, 0, :Dv] = np.nan                      # its output is never read
    oref, lref = O.lse_merge_packed(part.astype(np.float64))
    out, lse = pa.lse_merge(to_dev(part), out_dtype=dtype)
    torch.cuda.synchronize()
    check_close(to_f64(out), oref, "merge out", atol=1e-5 if dtype == torch.float32 else 1e-2,
                rtol=1e-5 if dtype == torch.float32 else 1e-2)
    check_lse(lse.cpu().numpy().astype(np.float64), lref, "merge lse", tol=1e-5)


def test_lse_merge_fig5c():
    """Figure 5c on the device: (15, a + ln 2) with (35, a + ln 4) -> 85/3."""
    say("lse_merge fig5c")
    a = 0.75
    part = np.array([[[[15.0, a + math.log(2)], [35.0, a + math.log(4)]]]], dtype=np.float32)
    out, lse = pa.lse_merge(to_dev(part))
    torch.cuda.synchronize()
    assert abs(float(out.item()) - 85.0 / 3.0) < 1e-4
    assert abs(float(lse.item()) - (a + math.log(6))) < 1e-5


# --------------------------------------------------- full-size workloads
@pytest.fixture(scope="module")
def llama():
    return W.llama_decode()


def test_llama_decode_full_size(llama):
    """64 requests, 32/8 heads, bf16; heuristic splits (as the bench runs it);
    every request against the oracle, the whole pool bit-exact."""
    b = llama
    say(f"decode llama3-8b full size, max_seq_len={b.max_seq_len}")
    cache_t, out, lse = _run_decode(b, num_splits=0)
    assert np.all(np.isfinite(out))
    cache_ref, oref, lref = _oracle_decode(b)
    check_close(out, oref, "llama decode out")
    check_lse(lse, lref, "llama decode lse")
    assert np.array_equal(bits(cache_t), cache_ref)


@pytest.fixture(scope="module")
def longctx():
    """The long-context batch and its oracle result (computed once: about a
    minute and a half of CPU work, shared by both schedules' tests)."""
    b = W.long_context_decode()
    say("long-context oracle")
    _, oref, lref = _oracle_decode(b)
    return b, oref, lref


def test_long_context_decode_full_size(longctx):
    """4 x 131072 keys, 64/8 heads, 256 splits; every request against the oracle."""
    b, oref, lref = longctx
    say("decode long-context full size (256 splits)")
    assert pa.num_kv_splits(b.max_seq_len, 256) == 256
    _, out, lse = _run_decode(b, num_splits=256)
    assert np.all(np.isfinite(out))
    check_close(out, oref, "long-context out")
    check_lse(lse, lref, "long-context lse")


def test_long_context_balanced_full_size(longctx):
    """The same batch on the automatic (token-balanced) schedule, as the bench
    runs it; every request against the oracle."""
    b, oref, lref = longctx
    say("balanced long-context full size")
    _, out, lse = _run_decode(b, num_splits=0)
    assert np.all(np.isfinite(out))
    check_close(out, oref, "long-context balanced out")
    check_lse(lse, lref, "long-context balanced lse")


def test_two_stage_decode_matches_one_call():
    """out = NULL runs stage 1 only; pa_lse_merge over its partials gives the
    one-call result (the pages' two-stage split-KV form)."""
    say("decode two-stage")
    b = _small(21, [700, 33, 1, 2000], 32, 8, W.BF16)
    cache_t, out1, lse1 = _run_decode(b, num_splits=5)
    part = pa.decode(to_dev(b.q), cache_t, to_dev(b.block_table), to_dev(b.seq_lens),
                     b.max_seq_len, b.scale, num_splits=5, stage1_only=True)
    out2, lse2 = pa.lse_merge(part, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert part.shape == (4, 32, 5, 129)
    assert np.array_equal(to_f64(out2), out1)
    assert np.array_equal(lse2.cpu().numpy().astype(np.float64), lse1)
    # the partials themselves: each non-empty split against the oracle's split
    cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
    p = part.cpu().numpy().astype(np.float64)
    P = -(-b.max_seq_len // 5)
    P = -(-P // b.block_size) * b.block_size
    for r in range(4):
        K, V = O.gather_kv(cache, b.block_table[r], int(b.seq_lens[r]))
        q = O.to_f64(b.q[r:r + 1])
        for s in range(5):
            lo, hi = s * P, min(int(b.seq_lens[r]), (s + 1) * P)
            if lo >= hi:
                assert np.all(p[r, :, s, 128] == -np.inf)
                continue
            o, l = O.partial_attention(q, K, V, b.scale, lo, hi, None)
            check_close(p[r, :, s, :128], o[0], f"partial r={r} s={s}", atol=2e-3, rtol=2e-3)
            check_lse(p[r, :, s, 128], l[0], f"partial lse r={r} s={s}")
