"""The mixed-batch planner on the host (pa_plan_mixed) and the run's argument
checks (pa_mixed_attention): no device work, these run without a GPU.

The plan splits a batch into its leading one-row (decode) requests and the
rest, the split a runner that orders decode requests first hands to a
backend ("Attention Backends", "Two kernels inside one attention call"), and
fixes the decode group's schedule the way pa_decode's automatic choice does
("第 1 章 注意力后端", §4.2 Plan/Run)."""
import ctypes as C
import math
import os

import numpy as np
import pytest

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.library_path()):
        pytest.fail("libpa.so is not built: run `python -m paged_kv_attention_pa_amd.build`")
    return pa.library()


def _qsl(q_lens):
    return [0] + list(np.cumsum(q_lens).astype(int))


def _expected_decode_schedule(nd, max_len, hq, hkv, bs, cus):
    """The decode group's schedule as the header states it: n =
    pa_num_kv_splits (the oracle's copy of the rule); one pass if the
    block-aligned split of max_len keys needs one split, else token-balanced
    ranges (1, 2, 4 or a multiple of 8 KV heads) or n splits."""
    if nd == 0:
        return 1, 0, 0
    n = O.num_kv_splits(max_len, cus)
    P = math.ceil(math.ceil(max_len / n) / bs) * bs
    if math.ceil(max_len / P) <= 1:
        return 1, 0, 0
    if hkv in (1, 2, 4) or hkv % 8 == 0:
        nr = pa.decode_balanced_num_ranges(hkv, cus)
        return n, nr, pa.decode_balanced_workspace_bytes(nd, hq, 128, nr)
    return n, 0, pa.decode_workspace_bytes(nd, hq, 128, n)


@pytest.mark.parametrize("q_lens,seq,hq,hkv,cus", [
    ([1, 1, 1, 70, 1, 200, 0], [900, 17, 5000, 100, 3000, 250, 12], 32, 8, 256),
    ([1] * 10, list(range(600, 6600, 600)), 32, 8, 256),     # decode only, balanced
    ([1, 1], [40, 100], 8, 2, 256),                            # decode only, one pass
    ([5, 1, 1], [5, 9, 9], 8, 8, 80),                          # prefill only (first L != 1)
    ([1, 1, 300], [20000, 70000, 900], 12, 6, 256),            # 6 KV heads: n splits
    ([1, 0, 1], [8, 0, 4], 4, 4, 256),                         # empty request ends the decode run
])
def test_plan_fields(lib, q_lens, seq, hq, hkv, cus):
    plan = pa.plan_mixed(_qsl(q_lens), seq, hq, hkv, 128, 16, 4096 // 16 * 32, cus)
    nd = 0
    while nd < len(q_lens) and q_lens[nd] == 1:
        nd += 1
    assert plan.num_seqs == len(q_lens)
    assert plan.num_tokens == sum(q_lens)
    assert plan.num_decode == nd
    assert plan.prefill_tokens == sum(q_lens[nd:])
    assert plan.max_decode_seq_len == (max(seq[:nd]) if nd else 0)
    assert plan.max_query_len == (max(q_lens[nd:]) if nd < len(q_lens) else 0)
    assert plan.max_seq_len == (max(seq[nd:]) if nd < len(q_lens) else 0)
    assert (plan.num_q_heads, plan.num_kv_heads, plan.head_dim, plan.block_size) == (hq, hkv, 128, 16)
    splits, ranges, ws = _expected_decode_schedule(nd, plan.max_decode_seq_len, hq, hkv, 16, cus)
    assert (plan.decode_splits, plan.decode_ranges, plan.workspace_bytes) == (splits, ranges, ws)


def test_plan_of_the_mixed_workload(lib):
    b = W.mixed_batch()
    plan = pa.plan_mixed(b.query_start_loc, b.seq_lens, 32, 8, 128, 16, b.block_table.shape[1], 256)
    assert plan.num_decode == 64 and plan.num_seqs == 68
    assert plan.prefill_tokens == int(b.q_lens[64:].sum())
    assert plan.decode_ranges == 256 and plan.decode_splits > 1


def test_plan_empty_batch(lib):
    plan = pa.plan_mixed([0], [], 32, 8, 128, 16, 64, 256)
    assert (plan.num_seqs, plan.num_tokens, plan.num_decode, plan.workspace_bytes) == (0, 0, 0, 0)


def _raw_plan(lib, qsl, seq, hq=32, hkv=8, d=128, bs=16, maxb=64, cus=256):
    plan = pa.MixedPlan()
    plan.num_seqs = 77   # must be cleared on error
    a = (C.c_int32 * max(len(qsl), 1))(*qsl)
    s = (C.c_int32 * max(len(seq), 1))(*seq)
    st = lib.pa_plan_mixed(a, s, len(seq), hq, hkv, d, bs, maxb, cus, C.byref(plan))
    return st, plan


@pytest.mark.parametrize("qsl,seq,kw,status", [
    ([1, 2], [5], {}, INVALID),                    # query_start_loc[0] != 0
    ([0, 3, 2], [5, 5], {}, INVALID),              # decreasing
    ([0, 3], [2], {}, INVALID),                    # more query rows than keys
    ([0, 1], [64 * 16 + 1], {}, INVALID),          # longer than the table addresses
    ([0, 1], [5], dict(d=64), UNSUPPORTED),
    ([0, 1], [5], dict(hq=24, hkv=8), UNSUPPORTED),   # group 3
    ([0, 1], [5], dict(hq=30, hkv=8), INVALID),
    ([0, 1], [5], dict(bs=8), INVALID),
    ([0, 1], [5], dict(maxb=0), INVALID),
    ([0, 1], [5], dict(cus=-1), INVALID),
])
def test_plan_validation(lib, qsl, seq, kw, status):
    st, plan = _raw_plan(lib, qsl, seq, **kw)
    assert st == status
    assert pa.last_error() != ""
    assert plan.num_seqs == 0


def test_plan_requires_host_copies():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU tensors here")
    with pytest.raises(ValueError):
        pa.plan_mixed(torch.zeros(2, dtype=torch.int32, device="cuda"), [1], 8, 8, 128, 16, 4)


def _run(lib, plan, **kw):
    a = dict(dtype=1, q=1 << 20, k=None, v=None, cache=1 << 21, nb=100, table=1 << 22,
             slots=None, qsl=1 << 23, seq=1 << 24, scale=0.1, ws=None, wsb=0, out=1 << 25,
             lse=None)
    a.update(kw)
    return lib.pa_mixed_attention(None if plan is None else C.byref(plan), a["dtype"], a["q"],
                                  a["k"], a["v"], a["cache"], a["nb"], a["table"], a["slots"],
                                  a["qsl"], a["seq"], a["scale"], a["ws"], a["wsb"], a["out"],
                                  a["lse"], None)


def test_run_validation(lib):
    # 4 decode requests long enough for the balanced schedule, then 1 chunk
    plan = pa.plan_mixed(_qsl([1, 1, 1, 1, 50]), [4000, 900, 70, 1000, 60], 32, 8, 128, 16, 256,
                         256)
    assert plan.decode_ranges > 0 and plan.workspace_bytes > 0
    need = plan.workspace_bytes
    assert _run(lib, None) == INVALID
    assert _run(lib, plan, dtype=0) == UNSUPPORTED                   # fp32
    assert _run(lib, plan, scale=float("nan")) == INVALID
    assert _run(lib, plan, ws=None) == WORKSPACE
    assert _run(lib, plan, ws=1 << 26, wsb=need - 1) == WORKSPACE
    assert _run(lib, plan, ws=(1 << 26) + 4, wsb=need) == INVALID   # misaligned workspace
    assert _run(lib, plan, ws=1 << 26, wsb=need, k=1 << 27) == INVALID   # k without v
    assert _run(lib, plan, ws=1 << 26, wsb=need, slots=1 << 27) == INVALID
    assert _run(lib, plan, ws=1 << 26, wsb=need, table=None) == INVALID
    assert _run(lib, plan, ws=1 << 26, wsb=need, qsl=None) == INVALID
    assert _run(lib, plan, ws=1 << 26, wsb=need, nb=0) == INVALID
    bad = pa.MixedPlan.from_buffer_copy(plan)
    bad.num_decode = bad.num_seqs + 1
    assert _run(lib, bad, ws=1 << 26, wsb=need) == INVALID
    bad = pa.MixedPlan.from_buffer_copy(plan)
    bad.decode_splits = 0
    assert _run(lib, bad, ws=1 << 26, wsb=need) == INVALID


def test_run_empty_batch_is_noop(lib):
    plan = pa.plan_mixed([0], [], 32, 8, 128, 16, 64, 256)
    assert _run(lib, plan, q=None, out=None, qsl=None, seq=None) == 0
    assert pa.last_error() == ""
