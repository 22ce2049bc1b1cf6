#!/usr/bin/env python3
"""Throughput of the paged-attention hot path on one MI355X (gfx950).

A step is one pass of the whole path over one synthetic batch: the new-token
cache write, the attention kernel(s) and, for split-KV decode, the LSE merge.
The headline line measures the Llama-3-8B-shaped GQA decode (64 requests,
seq_len U[512, 8192], 32 q / 8 kv heads, d=128, bf16, block 16) in HBM GB/s;
the other workloads (tiny fp32 decode, chunked prefill, long-context decode,
MLA decode, a mixed prefill + decode batch, a batch sharing a prefix, GQA and
MLA decode and chunked prefill over FP8 caches, MLA prefill) are measured the same way and
reported under "workloads".  Inputs are generated on the host by ``workloads.py`` (seeded),
uploaded once, and resident in HBM before any timed region.

Timing: W untimed warm-up steps, then K steps bracketed by
torch.cuda.synchronize() (wall clock); the dominant kernel of each workload
is also timed alone with HIP events on the stream it is launched on (the
library launches on torch's current stream).  The CPU baseline is the float64
oracle on a bounded sample of each of the five configurations (tiny decode,
Llama-3-8B decode, chunked prefill, long-context decode, MLA decode) on the
host's cores; the headline line carries the Llama-3-8B one.  Beside the
automatic schedule, the decode and MLA workloads are also timed at fixed
split counts, and the headline batch with an identity-like block table.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME ...]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HEADLINE = "llama3_8b_gqa_decode_bf16"
METRIC = "paged decode HBM GB/s (% of peak); prefill & MLA TFLOP/s (% of MFMA peak)"
CSRC = os.path.join(ROOT, "paged_kv_attention_pa_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha(fname: str) -> str:
    h = hashlib.sha256()
    for f in (fname, "pa_device.hpp", "launch.hpp", "balanced.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# one workload: inputs on the device, the step, the dominant kernel alone
# --------------------------------------------------------------------------

class Case:
    def __init__(self, name, step, kernel, step_bytes, step_flops, kern_bytes, kern_flops,
                 bound, kernel_name, source, info, sweep=None):
        self.name, self.step, self.kernel = name, step, kernel
        self.step_bytes, self.step_flops = step_bytes, step_flops
        self.kern_bytes, self.kern_flops = kern_bytes, kern_flops
        self.bound, self.kernel_name, self.source, self.info = bound, kernel_name, source, info
        # optional: {label: (num_splits, step function)} timed beside the case
        self.sweep = sweep


def _dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def gqa_decode_case(b, num_splits, name, split_sweep=False):
    import torch
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache, q = _dev(b.cache), _dev(b.q)
    bt, sl = _dev(b.block_table), _dev(b.seq_lens)
    kn, vn, sm = _dev(b.k_new), _dev(b.v_new), _dev(b.slot_mapping)
    cus = pa.device_num_cus()
    n = num_splits or pa.decode_num_kv_splits(b.num_seqs, b.num_kv_heads, b.max_seq_len, cus)
    g = b.num_q_heads // b.num_kv_heads
    # the automatic schedule (num_splits = 0) of bf16 decode over more than one
    # split's worth of keys is the token-balanced one
    balanced = num_splits == 0 and n > 1 and b.dtype == W.BF16
    if balanced:
        nr = pa.decode_balanced_num_ranges(b.num_kv_heads, cus)
        wsb = pa.decode_balanced_workspace_bytes(b.num_seqs, b.num_q_heads, b.head_dim, nr)
    else:
        wsb = pa.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.head_dim, n)
    ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        pa.decode(q, cache, bt, sl, b.max_seq_len, b.scale, k=kn, v=vn, slot_mapping=sm,
                  num_splits=num_splits, workspace=ws, out=out, lse=lse)

    if balanced:
        def kernel():
            pa.decode_balanced(q, cache, bt, sl, b.scale, num_ranges=nr, workspace=ws, out=out,
                               lse=lse, merge=False)
        kname = f"decode_balanced_kernel<{g}, false>"
        grid = f"{nr} token ranges x {min(b.num_kv_heads, 8)} waves (one per KV head)"
        source = "decode_balanced.hip"
    else:
        def kernel():
            pa.decode(q, cache, bt, sl, b.max_seq_len, b.scale, num_splits=n, workspace=ws,
                      stage1_only=True)
        kname = (f"decode_mfma_kernel<{g}>" if b.dtype == W.BF16
                 else f"decode_split_kernel<false, {g}>")
        grid = f"{b.num_seqs}x{b.num_kv_heads}x{n} work-groups of 256"
        source = "decode.hip"

    by = W.gqa_bytes(b)
    kb = by["kv"] + by["q"] + by["meta"] - b.num_tokens * 8   # attention kernel: KV, q, table walk
    fl = W.gqa_flops(b)
    info = {"num_seqs": b.num_seqs, "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads,
            "head_dim": b.head_dim, "block_size": b.block_size, "dtype": b.dtype,
            "max_seq_len": b.max_seq_len, "total_keys": int(b.seq_lens.sum()),
            "schedule": "token-balanced ranges" if balanced else f"{n} splits per request",
            "grid": grid}
    sweep = None
    if split_sweep:
        # the pages' fixed partition at several split counts: unsplit, two,
        # their heuristic (max_seq_len / 512, capped at 2 x CUs) and the cap
        counts = {"1": 1, "2": 2, "heuristic": pa.num_kv_splits(b.max_seq_len, cus),
                  "max (2 x CUs)": 2 * cus}
        sweep = {}
        for label, ns in counts.items():
            need = pa.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.head_dim, ns)
            wsn = torch.empty(max(1, need // 4), dtype=torch.float32, device="cuda")

            def run(ns=ns, wsn=wsn):
                pa.decode(q, cache, bt, sl, b.max_seq_len, b.scale, k=kn, v=vn, slot_mapping=sm,
                          num_splits=ns, workspace=wsn, out=out, lse=lse)
            sweep[label] = (ns, run)
    c = Case(name, step, kernel, by["total"], fl, kb, fl, "hbm", kname, source, info, sweep)
    c.batch = b
    return c


def prefill_case(b, name):
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache, q = _dev(b.cache), _dev(b.q)
    bt, sl, qsl = _dev(b.block_table), _dev(b.seq_lens), _dev(b.query_start_loc)
    kn, vn, sm = _dev(b.k_new), _dev(b.v_new), _dev(b.slot_mapping)
    import torch
    out = torch.empty_like(q)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        pa.prefill_varlen(q, cache, bt, qsl, sl, b.max_query_len, b.max_seq_len, b.scale,
                          k=kn, v=vn, slot_mapping=sm, out=out, lse=lse)

    def kernel():
        pa.prefill_varlen(q, cache, bt, qsl, sl, b.max_query_len, b.max_seq_len, b.scale,
                          out=out, lse=lse)

    by = W.gqa_bytes(b)
    kb = by["total"] - by["write"]
    fl = W.gqa_flops(b)
    info = {"num_seqs": b.num_seqs, "num_tokens": b.num_tokens, "num_q_heads": b.num_q_heads,
            "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": b.block_size,
            "max_query_len": b.max_query_len, "max_seq_len": b.max_seq_len, "causal": True,
            "grid": "ceil(max_q/256) x num_seqs x Hq work-groups of 512 (two 4-wave groups "
                    "alternating MFMA and softmax half-periods)"}
    c = Case(name, step, kernel, by["total"], fl, kb, fl, "mfma", "prefill_pp_kernel<2>",
             "prefill.hip", info)
    c.batch = b
    return c


def mla_case(b, name):
    import torch
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache = _dev(b.cache)
    qn, qp = _dev(b.q_nope), _dev(b.q_pe)
    bt, sl = _dev(b.block_table), _dev(b.seq_lens)
    kc, kp, sm = _dev(b.kv_c_new), _dev(b.k_pe_new), _dev(b.slot_mapping)
    # automatic schedule: token-balanced ranges, one per compute unit
    nr = pa.device_num_cus()
    wsb = pa.decode_balanced_workspace_bytes(b.num_seqs, b.num_heads, b.kv_lora_rank, nr)
    ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device="cuda")
    out = torch.empty((b.num_seqs, b.num_heads, b.kv_lora_rank), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b.num_seqs, b.num_heads), dtype=torch.float32, device="cuda")

    def step():
        pa.mla_decode(qn, qp, cache, bt, sl, b.max_seq_len, b.scale, kv_c=kc, k_pe=kp,
                      slot_mapping=sm, num_splits=0, workspace=ws, out=out, lse=lse)

    def kernel():
        pa.mla_decode_balanced(qn, qp, cache, bt, sl, b.scale, num_ranges=nr, workspace=ws,
                               out=out, lse=lse, merge=False)

    by = W.mla_bytes(b)
    kb = by["kv"] + by["q"] + by["meta"] - b.num_seqs * 8
    fl = W.mla_flops(b)
    info = {"num_seqs": b.num_seqs, "num_heads": b.num_heads, "kv_lora_rank": b.kv_lora_rank,
            "rope_dim": b.rope_dim, "block_size": b.block_size, "max_seq_len": b.max_seq_len,
            "total_keys": int(b.seq_lens.sum()), "schedule": "token-balanced ranges",
            "grid": f"{nr} token ranges x 4 waves (32 heads each)"}
    # fixed partitions: unsplit, 2, 4, the library's MLA rule (enough splits to
    # cover the CUs about twice) and the pages' max_seq_len / 512
    counts = {"1": 1, "2": 2, "4": 4,
              "mla rule": pa.mla_num_kv_splits(b.num_seqs, b.max_seq_len, nr),
              "heuristic (max_seq_len / 512)": pa.num_kv_splits(b.max_seq_len, nr)}
    sweep = {}
    for label, ns in counts.items():
        need = pa.decode_workspace_bytes(b.num_seqs, b.num_heads, b.kv_lora_rank, ns)
        wsn = torch.empty(max(1, need // 4), dtype=torch.float32, device="cuda")

        def run(ns=ns, wsn=wsn):
            pa.mla_decode(qn, qp, cache, bt, sl, b.max_seq_len, b.scale, kv_c=kc, k_pe=kp,
                          slot_mapping=sm, num_splits=ns, workspace=wsn, out=out, lse=lse)
        sweep[label] = (ns, run)
    c = Case(name, step, kernel, by["total"], fl, kb, fl, "mfma", "mla_kernel<true, false, 512>",
             "mla_decode.hip", info, sweep)
    c.batch = b
    return c


def mixed_case(b, name):
    """A planned mixed batch: decode group (token-balanced schedule) then the
    prefill group, one plan.  Its roofline is a time: the decode group's
    algorithmic bytes at peak HBM bandwidth plus the prefill group's flops at
    peak MFMA rate, the two kernels running one after the other."""
    import torch
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache, q = _dev(b.cache), _dev(b.q)
    bt, sl, qsl = _dev(b.block_table), _dev(b.seq_lens), _dev(b.query_start_loc)
    kn, vn, sm = _dev(b.k_new), _dev(b.v_new), _dev(b.slot_mapping)
    plan = pa.plan_mixed(b.query_start_loc, b.seq_lens, b.num_q_heads, b.num_kv_heads,
                         b.head_dim, b.block_size, b.block_table.shape[1])
    ws = torch.empty(max(1, (plan.workspace_bytes + 3) // 4), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        pa.mixed_attention(plan, q, cache, bt, qsl, sl, b.scale, k=kn, v=vn, slot_mapping=sm,
                           workspace=ws, out=out, lse=lse)

    def kernel():
        pa.mixed_attention(plan, q, cache, bt, qsl, sl, b.scale, workspace=ws, out=out, lse=lse)

    nd = plan.num_decode
    e, row = b.elem_bytes, b.num_kv_heads * b.head_dim * b.elem_bytes
    dec_bytes = (int(b.seq_lens[:nd].sum()) * row * 2 + 2 * nd * b.num_q_heads * b.head_dim * e
                 + int(((b.seq_lens[:nd].astype(int) + b.block_size - 1) // b.block_size).sum()) * 4)
    pf_flops = 0
    for L, S in zip(b.q_lens[nd:], b.seq_lens[nd:]):
        L, S = int(L), int(S)
        pf_flops += 2 * (L * (S - L) + L * (L + 1) // 2) * b.num_q_heads * 2 * b.head_dim
    by = W.gqa_bytes(b)
    case = Case(name, step, kernel, by["total"], W.gqa_flops(b), by["total"] - by["write"],
                W.gqa_flops(b), "hbm+mfma", "decode_balanced_kernel + merge + prefill_pp_kernel",
                "api.cpp",
                {"num_seqs": b.num_seqs, "num_decode": nd, "prefill_tokens": plan.prefill_tokens,
                 "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads,
                 "head_dim": b.head_dim, "block_size": b.block_size,
                 "max_decode_seq_len": plan.max_decode_seq_len,
                 "max_query_len": plan.max_query_len, "max_seq_len": plan.max_seq_len,
                 "decode_schedule": f"{plan.decode_ranges} token-balanced ranges"
                 if plan.decode_ranges else f"{plan.decode_splits} splits",
                 "decode_bytes": dec_bytes, "prefill_flops": pf_flops})
    case.roof_s = dec_bytes / (PEAK_HBM_GBS * 1e9) + pf_flops / (PEAK_BF16_TFLOPS * 1e12)
    return case


def cascade_case(b, name):
    """A batch whose requests share their first pages, run as a cascade (the
    prefix once for every query row, each request's own keys, the merge).
    Priced against HBM: the prefix's K/V counted once, each request's own
    K/V once.  The plain decode of the same batch (the prefix read once per
    request) is timed beside it."""
    import numpy as np
    import torch
    import paged_kv_attention_pa_amd as pa
    cache, q = _dev(b.cache), _dev(b.q)
    bt, sl, qsl = _dev(b.block_table), _dev(b.seq_lens), _dev(b.query_start_loc)
    kn, vn, sm = _dev(b.k_new), _dev(b.v_new), _dev(b.slot_mapping)
    P = b.meta["prefix_blocks"]
    plan = pa.plan_cascade(b.query_start_loc, b.seq_lens, P, b.num_q_heads, b.num_kv_heads,
                           b.head_dim, b.block_size, b.block_table.shape[1])
    ws = torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        pa.cascade_attention(plan, q, cache, bt, qsl, sl, b.scale, k=kn, v=vn, slot_mapping=sm,
                             workspace=ws, out=out, lse=lse)

    def kernel():
        pa.cascade_attention(plan, q, cache, bt, qsl, sl, b.scale, workspace=ws, out=out, lse=lse)

    # the plain path over the same batch, for comparison
    cus = pa.device_num_cus()
    nr = pa.decode_balanced_num_ranges(b.num_kv_heads, cus)
    pws = torch.empty(max(1, pa.decode_balanced_workspace_bytes(b.num_seqs, b.num_q_heads,
                                                                b.head_dim, nr)),
                      dtype=torch.uint8, device="cuda")
    plain_s = time_kernel_events(
        lambda: pa.decode(q, cache, bt, sl, b.max_seq_len, b.scale, workspace=pws, out=out,
                          lse=lse), 20, 5)

    e = b.elem_bytes
    row = b.num_kv_heads * b.head_dim * e
    Lp = P * b.block_size
    own = b.seq_lens.astype(np.int64) - Lp
    kv = (Lp + int(own.sum())) * row * 2
    nblk = P + int(((own + b.block_size - 1) // b.block_size).sum())
    qo = 2 * b.q.size * e + b.q.shape[0] * b.q.shape[1] * 4
    kb = kv + qo + nblk * 4 + b.num_seqs * 8
    wr = (b.k_new.size + b.v_new.size) * e * 2
    fl = 2 * b.num_q_heads * 2 * b.head_dim * int(b.seq_lens.sum())
    return Case(name, step, kernel, kb + wr + b.num_tokens * 8, fl, kb, fl, "hbm",
                "suffix decode + prefix pass + merges", "prefill.hip",
                {"num_seqs": b.num_seqs, "num_q_heads": b.num_q_heads,
                 "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                 "block_size": b.block_size, "prefix_len": Lp,
                 "own_keys": "U[512,4096]", "prefix_splits": plan.prefix_splits,
                 "split_keys": plan.split_keys,
                 "plain_decode_ms": round(plain_s * 1e3, 4),
                 "plain_decode_reads_GB": round((int(b.seq_lens.sum()) * row * 2) / 1e9, 3)})


def fp8_decode_case(b, name):
    """Decode over an FP8 (E4M3) cache: write + token-balanced decode +
    merge.  The timed kernel is the whole decode call (decode kernel and
    segment merge), priced against HBM with one byte per cached element."""
    import torch
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache = torch.from_numpy(b.cache).cuda()
    q = _dev(b.q)
    bt, sl = _dev(b.block_table), _dev(b.seq_lens)
    kn, vn, sm = _dev(b.k_new), _dev(b.v_new), _dev(b.slot_mapping)
    cus = pa.device_num_cus()
    nr = pa.decode_balanced_num_ranges(b.num_kv_heads, cus)
    ws = torch.empty(max(1, pa.decode_balanced_workspace_bytes(b.num_seqs, b.num_q_heads,
                                                               b.head_dim, nr) // 4),
                     dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        pa.decode_fp8(q, cache, bt, sl, b.scale, b.k_scale, b.v_scale, k=kn, v=vn,
                      slot_mapping=sm, num_ranges=nr, workspace=ws, out=out, lse=lse)

    def kernel():
        pa.decode_fp8(q, cache, bt, sl, b.scale, b.k_scale, b.v_scale, num_ranges=nr,
                      workspace=ws, out=out, lse=lse)

    by = W.gqa_bytes(b)
    kb = by["kv"] + by["q"] + by["meta"] - b.num_tokens * 8
    fl = W.gqa_flops(b)
    g = b.num_q_heads // b.num_kv_heads
    info = {"num_seqs": b.num_seqs, "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads,
            "head_dim": b.head_dim, "block_size": b.block_size, "cache_dtype": "fp8_e4m3",
            "k_scale": b.k_scale, "v_scale": b.v_scale, "max_seq_len": b.max_seq_len,
            "total_keys": int(b.seq_lens.sum()), "schedule": "token-balanced ranges",
            "timed": "decode kernel + segment merge"}
    return Case(name, step, kernel, by["total"], fl, kb, fl, "hbm",
                f"decode_balanced_kernel<{g}, true> + merge", "decode_balanced.hip", info)


def mla_fp8_case(b, name):
    """MLA decode over an FP8 latent cache: write + balanced decode + merge;
    the timed kernel is the decode call (decode kernel and segment merge),
    priced against the bf16 MFMA peak (the products run on bf16 MFMAs after
    the tiles are widened)."""
    import torch
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache = torch.from_numpy(b.cache).cuda()
    qn, qp = _dev(b.q_nope), _dev(b.q_pe)
    bt, sl = _dev(b.block_table), _dev(b.seq_lens)
    kc, kp, sm = _dev(b.kv_c_new), _dev(b.k_pe_new), _dev(b.slot_mapping)
    nr = pa.device_num_cus()
    wsb = pa.decode_balanced_workspace_bytes(b.num_seqs, b.num_heads, b.kv_lora_rank, nr)
    ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device="cuda")
    out = torch.empty((b.num_seqs, b.num_heads, b.kv_lora_rank), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b.num_seqs, b.num_heads), dtype=torch.float32, device="cuda")

    def step():
        pa.mla_decode_fp8(qn, qp, cache, bt, sl, b.scale, b.kv_scale, kv_c=kc, k_pe=kp,
                          slot_mapping=sm, num_ranges=nr, workspace=ws, out=out, lse=lse)

    def kernel():
        pa.mla_decode_fp8(qn, qp, cache, bt, sl, b.scale, b.kv_scale, num_ranges=nr, workspace=ws,
                          out=out, lse=lse)

    by = W.mla_bytes(b)
    kb = by["kv"] + by["q"] + by["meta"] - b.num_seqs * 8
    fl = W.mla_flops(b)
    info = {"num_seqs": b.num_seqs, "num_heads": b.num_heads, "kv_lora_rank": b.kv_lora_rank,
            "rope_dim": b.rope_dim, "block_size": b.block_size, "cache_dtype": "fp8_e4m3",
            "kv_scale": b.kv_scale, "max_seq_len": b.max_seq_len,
            "total_keys": int(b.seq_lens.sum()), "schedule": "token-balanced ranges",
            "timed": "decode kernel + segment merge"}
    return Case(name, step, kernel, by["total"], fl, kb, fl, "mfma",
                "mla_kernel<true, true, 512> + merge", "mla_decode.hip", info)


def mla_prefill_case(b, name):
    """MLA prefill in the multi-head form: latent write + key offsets +
    projection of every key + causal attention.  The timed call is the whole
    computation without the write (three kernels), priced against the bf16
    MFMA peak with the projection's and the attention's flops."""
    import torch
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache, q, w = _dev(b.cache), _dev(b.q), _dev(b.w_kv_b)
    bt, sl, qsl = _dev(b.block_table), _dev(b.seq_lens), _dev(b.query_start_loc)
    kc, kp, sm = _dev(b.kv_c_new), _dev(b.k_pe_new), _dev(b.slot_mapping)
    ws = torch.empty(pa.mla_prefill_workspace_bytes(b.num_seqs, b.total_keys, b.num_heads),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((b.num_tokens, b.num_heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b.num_tokens, b.num_heads), dtype=torch.float32, device="cuda")

    def step():
        pa.mla_prefill(q, cache, bt, qsl, sl, w, b.max_query_len, b.total_keys, b.scale, kv_c=kc,
                       k_pe=kp, slot_mapping=sm, workspace=ws, out=out, lse=lse)

    def kernel():
        pa.mla_prefill(q, cache, bt, qsl, sl, w, b.max_query_len, b.total_keys, b.scale,
                       workspace=ws, out=out, lse=lse)

    fl = W.mla_prefill_flops(b)
    kv = b.total_keys * 1152 + b.w_kv_b.size * 2 + b.q.size * 2 + b.num_tokens * b.num_heads * (256 + 4)
    info = {"num_seqs": b.num_seqs, "num_tokens": b.num_tokens, "num_heads": b.num_heads,
            "kv_lora_rank": 512, "rope_dim": 64, "qk_head_dim": 192, "v_head_dim": 128,
            "block_size": b.block_size, "total_keys": b.total_keys,
            "max_query_len": b.max_query_len, "projection_flops": fl["projection"],
            "attention_flops": fl["attention"], "timed": "key offsets + projection + attention"}
    return Case(name, step, kernel, kv, fl["total"], kv, fl["total"], "mfma",
                "mla_expand_kernel + mla_attn_kernel", "mla_prefill.hip", info)


def fp8_prefill_case(b, name):
    """Chunked prefill over an FP8 cache (write + attention); the timed kernel
    is the attention alone, priced against the bf16 MFMA peak."""
    import torch
    import paged_kv_attention_pa_amd as pa
    import workloads as W
    cache = torch.from_numpy(b.cache).cuda()
    q = _dev(b.q)
    bt, sl, qsl = _dev(b.block_table), _dev(b.seq_lens), _dev(b.query_start_loc)
    kn, vn, sm = _dev(b.k_new), _dev(b.v_new), _dev(b.slot_mapping)
    out = torch.empty_like(q)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        pa.prefill_varlen_fp8(q, cache, bt, qsl, sl, b.max_query_len, b.max_seq_len, b.scale,
                              b.k_scale, b.v_scale, k=kn, v=vn, slot_mapping=sm, out=out, lse=lse)

    def kernel():
        pa.prefill_varlen_fp8(q, cache, bt, qsl, sl, b.max_query_len, b.max_seq_len, b.scale,
                              b.k_scale, b.v_scale, out=out, lse=lse)

    by = W.gqa_bytes(b)
    fl = W.gqa_flops(b)
    info = {"num_seqs": b.num_seqs, "num_tokens": b.num_tokens, "num_q_heads": b.num_q_heads,
            "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": b.block_size,
            "cache_dtype": "fp8_e4m3", "k_scale": b.k_scale, "v_scale": b.v_scale,
            "max_query_len": b.max_query_len, "max_seq_len": b.max_seq_len, "causal": True}
    return Case(name, step, kernel, by["total"], fl, by["total"] - by["write"], fl, "mfma",
                "prefill_kernel<false, true>", "prefill.hip", info)


def build_cases(only):
    import workloads as W
    makers = {
        "tiny_gqa_decode_fp32": lambda: gqa_decode_case(W.tiny_decode(), 0, "tiny_gqa_decode_fp32"),
        HEADLINE: lambda: gqa_decode_case(W.llama_decode(), 0, HEADLINE, split_sweep=True),
        "chunked_prefill_varlen_bf16": lambda: prefill_case(W.chunked_prefill(),
                                                            "chunked_prefill_varlen_bf16"),
        "long_context_split_kv_decode_bf16": lambda: gqa_decode_case(
            W.long_context_decode(), 0, "long_context_split_kv_decode_bf16", split_sweep=True),
        W.IDENTITY_DECODE: lambda: gqa_decode_case(
            W.identity_layout(W.llama_decode(), W.IDENTITY_DECODE), 0, W.IDENTITY_DECODE),
        "mla_latent_decode_bf16": lambda: mla_case(W.mla_decode_batch(), "mla_latent_decode_bf16"),
        W.MIXED: lambda: mixed_case(W.mixed_batch(), W.MIXED),
        W.CASCADE: lambda: cascade_case(W.cascade_batch(), W.CASCADE),
        W.FP8_DECODE: lambda: fp8_decode_case(W.llama_decode_fp8(), W.FP8_DECODE),
        W.FP8_MLA: lambda: mla_fp8_case(W.mla_decode_fp8_batch(), W.FP8_MLA),
        W.MLA_PREFILL: lambda: mla_prefill_case(W.mla_prefill_batch(), W.MLA_PREFILL),
        W.FP8_PREFILL: lambda: fp8_prefill_case(W.chunked_prefill_fp8(), W.FP8_PREFILL),
    }
    names = [HEADLINE] + [n for n in makers if n != HEADLINE]
    if only is not None:   # exactly these (the line then reports the first one run)
        unknown = [n for n in only if n not in makers]
        if unknown:
            raise SystemExit(f"unknown workload(s) {unknown}; known: {names}")
        names = [n for n in names if n in only]
    for n in names:
        t = time.perf_counter()
        case = makers[n]()
        log(f"[bench] prepared {n} in {time.perf_counter() - t:.1f}s")
        yield case


# --------------------------------------------------------------------------
# timing
# --------------------------------------------------------------------------

def time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


_SPIN_RATE = None


def _hold_gpu(seconds):
    """Queue torch's bounded spin kernel for about ``seconds`` so that the
    launches issued next are all enqueued before the GPU reaches them: the
    events then time back-to-back kernels, not the host's launch gaps."""
    import torch
    global _SPIN_RATE
    if _SPIN_RATE is None:   # counter ticks per second of the spin kernel
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        torch.cuda._sleep(10_000_000)
        e.record()
        e.synchronize()
        _SPIN_RATE = 10_000_000 / max(s.elapsed_time(e) / 1e3, 1e-6)
    torch.cuda._sleep(int(seconds * _SPIN_RATE))


def time_kernel_events(fn, reps, warmup):
    """Average duration of one launch of ``fn``'s kernel, from HIP events
    recorded on torch's current stream (the stream the library launches on),
    with the launches queued behind a spin kernel so none waits on the host."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _hold_gpu(2 * host_s + 2e-3)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / 1000.0 / reps


def traffic_for(case):
    """HBM bytes per launch from the stored rocprofv3 counter runs, or None
    if they were taken on a different version of the kernel's source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(case.name)
    if not e or e.get("source_sha") != kernel_source_sha(case.source):
        return None
    return e.get("hbm_bytes_per_launch")


def roofline(case, kern_s):
    if case.bound == "hbm+mfma":
        # a time roofline: each group at its own roof, one after the other
        return {"bound": case.bound, "kernel": case.kernel_name,
                "achieved": round(kern_s * 1e3, 4), "peak": round(case.roof_s * 1e3, 4),
                "unit": "ms (measured vs roofline time)", "frac": round(case.roof_s / kern_s, 4),
                "traffic": None, "kernel_ms": round(kern_s * 1e3, 4),
                "algorithmic_bytes": int(case.kern_bytes), "algorithmic_flops": int(case.kern_flops),
                "kernel_GBps": round(case.kern_bytes / kern_s / 1e9, 1),
                "kernel_TFLOPs": round(case.kern_flops / kern_s / 1e12, 2)}
    if case.bound == "hbm":
        achieved = case.kern_bytes / kern_s / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    else:
        achieved = case.kern_flops / kern_s / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    # both roofs, for a reader placing the kernel against the ridge point
    # (MLA decode, about 230 flop/byte, sits on the HBM side of it)
    gbs = case.kern_bytes / kern_s / 1e9
    tfs = case.kern_flops / kern_s / 1e12
    return {"bound": case.bound, "kernel": case.kernel_name, "achieved": round(achieved, 2),
            "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": traffic_for(case), "kernel_ms": round(kern_s * 1e3, 4),
            "algorithmic_bytes": int(case.kern_bytes), "algorithmic_flops": int(case.kern_flops),
            "kernel_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "kernel_TFLOPs": round(tfs, 2), "mfma_frac": round(tfs / PEAK_BF16_TFLOPS, 4),
            "flop_per_byte": round(case.kern_flops / max(case.kern_bytes, 1), 1)}


# --------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of each of the five
# configurations, on the host's cores
# --------------------------------------------------------------------------

CPU_SAMPLES = {   # workload -> (kind, seconds of oracle work to aim for)
    "tiny_gqa_decode_fp32": ("decode", 2.0),
    HEADLINE: ("decode", 5.0),
    "chunked_prefill_varlen_bf16": ("prefill", 5.0),
    "long_context_split_kv_decode_bf16": ("decode", 5.0),
    "mla_latent_decode_bf16": ("mla", 5.0),
}


def _host_threads() -> int:
    """Threads the oracle's BLAS may use: the cores this process may run on,
    no more than the OMP_NUM_THREADS share when one is set."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ["OMP_NUM_THREADS"]))
    except (KeyError, ValueError):
        pass
    return max(1, n)


def cpu_baseline(name, case):
    """Time the oracle on a bounded sample of workload ``name``: the whole
    batch's cache write, then the attention of its requests in order until
    the time budget is spent (at least one request).  Reported in the unit of
    the workload's roofline: GB/s of the sampled requests' algorithmic bytes
    for decode, GFLOP/s of their flops for prefill and MLA."""
    import numpy as np
    import workloads as W
    import oracle.pa_oracle as O
    from threadpoolctl import threadpool_limits
    kind, budget = CPU_SAMPLES[name]
    make = {"tiny_gqa_decode_fp32": W.tiny_decode, HEADLINE: W.llama_decode,
            "chunked_prefill_varlen_bf16": W.chunked_prefill,
            "long_context_split_kv_decode_bf16": W.long_context_decode,
            "mla_latent_decode_bf16": W.mla_decode_batch}[name]
    b = getattr(case, "batch", None) or make()
    threads = _host_threads()
    done, work = 0, 0.0
    with threadpool_limits(limits=threads):
        tw = time.perf_counter()
        if kind == "mla":
            cache = O.cache_write_mla(b.cache, b.kv_c_new, b.k_pe_new, b.slot_mapping)
        else:
            cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
        t0 = time.perf_counter()
        write_s = t0 - tw
        for r in range(b.num_seqs):
            S = int(b.seq_lens[r])
            if kind == "decode":
                O.paged_decode(b.q, cache, b.block_table, b.seq_lens, b.scale, requests=[r])
                elem = 4 if b.dtype == W.F32 else 2
                work += S * 2 * b.num_kv_heads * b.head_dim * elem + 2 * b.num_q_heads * b.head_dim * elem
            elif kind == "prefill":
                O.paged_attention(b.q, cache, b.block_table, b.query_start_loc, b.seq_lens,
                                  b.scale, requests=[r])
                L = int(b.query_start_loc[r + 1] - b.query_start_loc[r])
                C = S - L
                work += 4.0 * b.head_dim * b.num_q_heads * (L * C + L * (L + 1) / 2)
            else:
                O.mla_decode(b.q_nope, b.q_pe, cache, b.block_table, b.seq_lens, b.scale,
                             requests=[r])
                work += 2.0 * b.num_heads * S * ((b.kv_lora_rank + b.rope_dim) + b.kv_lora_rank)
            done += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = time.perf_counter() - t0
    unit, value = ("GB/s", work / dt / 1e9) if kind == "decode" else ("GFLOP/s", work / dt / 1e9)
    return {"value": round(value, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2), "write_seconds": round(write_s, 2),
            "sample": f"float64 numpy oracle, {threads} BLAS threads: the attention of {done} of "
                      f"{b.num_seqs} requests (in order) over the cache after the batch's write "
                      f"(the write, {write_s:.2f} s, is timed apart and not in the rate)"}


# --------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", nargs="*", default=None,
                    help="run only these workloads (default: all, the headline first)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, --steps times "
                         "(the reference kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path is single-GPU by design (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": n * 4, "copy_bytes_written_per_launch": n * 4,
                          "launches": args.steps}), flush=True)
        return
    import paged_kv_attention_pa_amd as pa
    pa.library()   # fails loudly if the HIP library is missing

    results = {}
    head = None
    for case in build_cases(args.only):
        step_s = time_steps(case.step, args.steps, args.warmup)
        kern_s = time_kernel_events(case.kernel, args.steps, args.warmup)
        rl = roofline(case, kern_s)
        res = {
            "ms_per_step": round(step_s * 1e3, 4),
            "step_GBps": round(case.step_bytes / step_s / 1e9, 2),
            "step_TFLOPs": round(case.step_flops / step_s / 1e12, 3),
            "step_bytes": int(case.step_bytes), "step_flops": int(case.step_flops),
            "roofline": rl, "config": case.info,
        }
        if case.sweep:
            sw = {}
            for label, (ns, fn) in case.sweep.items():
                t = time_steps(fn, args.steps, args.warmup)
                sw[label] = {"num_splits": ns, "ms_per_step": round(t * 1e3, 4),
                             "step_GBps": round(case.step_bytes / t / 1e9, 2),
                             "step_TFLOPs": round(case.step_flops / t / 1e12, 3)}
                log(f"[bench]   {case.name} num_splits={ns} ({label}): {sw[label]['ms_per_step']} ms/step")
            sw["automatic (this line)"] = {"num_splits": 0, "ms_per_step": res["ms_per_step"],
                                           "step_GBps": res["step_GBps"],
                                           "step_TFLOPs": res["step_TFLOPs"]}
            res["num_splits_sweep"] = sw
        if not args.no_cpu_baseline and case.name in CPU_SAMPLES:
            res["cpu_baseline"] = cpu_baseline(case.name, case)
            log(f"[bench]   {case.name} cpu baseline: {res['cpu_baseline']['value']} "
                f"{res['cpu_baseline']['unit']} on {res['cpu_baseline']['cores']} threads")
        results[case.name] = res
        log(f"[bench] {case.name}: {res['ms_per_step']} ms/step, {res['step_GBps']} GB/s, "
            f"{res['step_TFLOPs']} TFLOP/s; kernel {rl['kernel']} {rl['kernel_ms']} ms = "
            f"{rl['achieved']} {rl['unit']} ({100 * rl['frac']:.1f}% of peak)")
        if head is None or case.name == HEADLINE:
            head = (case, step_s, rl)
        del case
        torch.cuda.empty_cache()

    case, step_s, rl = head
    line = {
        "metric": METRIC,
        "value": round(case.step_bytes / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, **results[case.name]["config"],
                   **({"seq_len": "U[512,8192]"} if case.name == HEADLINE else {}),
                   "parallelism": "single GPU"},
        "roofline": {k: rl[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "cpu_baseline": results[case.name].get("cpu_baseline"),
        "dominant_kernel": {k: rl[k] for k in ("kernel", "kernel_ms", "algorithmic_bytes")},
        "workloads": results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
