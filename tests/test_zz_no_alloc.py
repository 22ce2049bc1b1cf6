"""pa_decode_noalloc: the decode entry point whose partials live in the
library's own device array (for callers that cannot allocate).  It is called
through the C ABI and must give pa_decode's result bit for bit (same kernels,
same schedule) on two calls in a row, the second with a smaller batch, and
reject a batch whose workspace would not fit the array."""
import ctypes as C
import math

import numpy as np
import pytest

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa
import workloads as W

WORKSPACE = 3


def _noalloc_raw(b, dev, num_splits, out, lse):
    lib = pa.library()
    q, cache, table, seq = dev["q"], dev["cache"], dev["table"], dev["seq"]
    k, v, slots = dev["k"], dev["v"], dev["slots"]
    return lib.pa_decode_noalloc(1, q.data_ptr(), k.data_ptr(), v.data_ptr(), cache.data_ptr(),
                                 cache.shape[0], b.block_size, table.data_ptr(), table.shape[1],
                                 slots.data_ptr(), seq.data_ptr(), len(b.seq_lens),
                                 int(b.max_seq_len), b.q.shape[1], b.cache.shape[3],
                                 b.cache.shape[4], float(b.scale), int(num_splits),
                                 out.data_ptr(), lse.data_ptr(), None)


def test_noalloc_rejects_a_workspace_beyond_the_array():
    """300 requests x 64 heads x 512 splits need ~5 GB of partials: refused on
    the host before anything is launched (explicit splits need no device)."""
    lib = pa.library()
    st = lib.pa_decode_noalloc(1, 1 << 20, None, None, 1 << 21, 100000, 16, 1 << 22, 8192,
                               None, 1 << 23, 300, 131072, 64, 8, 128, 0.1, 512, 1 << 24,
                               None, None)
    assert st == WORKSPACE
    assert "PA_NOALLOC_SCRATCH_BYTES" in pa.last_error()
    assert lib.pa_decode_noalloc(1, 1 << 20, None, None, 1 << 21, 1000, 16, 1 << 22, 64,
                                 None, 1 << 23, 4, 1000, 32, 8, 128, 0.1, 2, None, None,
                                 None) == 1            # out is required


@pytest.mark.gpu
def test_noalloc_matches_pa_decode_on_two_calls():
    import torch
    from gpu_util import bits, check_close, check_lse, say, to_dev, to_f64

    def dev_of(b):
        return {"q": to_dev(b.q), "cache": to_dev(b.cache), "table": to_dev(b.block_table),
                "seq": to_dev(b.seq_lens), "k": to_dev(b.k_new), "v": to_dev(b.v_new),
                "slots": to_dev(b.slot_mapping)}

    big = W.make_gqa(501, np.ones(48, np.int64),
                     np.random.default_rng(5).integers(512, 8193, 48), 32, 8, 128, 16, W.BF16,
                     scale=1.0 / math.sqrt(128))
    small = W.make_gqa(502, np.ones(5, np.int64), [17, 700, 3000, 1, 64], 32, 8, 128, 16, W.BF16,
                       scale=1.0 / math.sqrt(128))
    for name, b, splits in (("48 requests, automatic schedule", big, 0),
                            ("5 requests, automatic schedule", small, 0),
                            ("48 requests, 7 splits", big, 7),
                            ("5 requests, 3 splits", small, 3)):
        say(f"noalloc {name}")
        d1, d2 = dev_of(b), dev_of(b)
        B, Hq = b.q.shape[0], b.q.shape[1]
        out_n = torch.empty_like(d1["q"])
        lse_n = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=out_n.device)
        st = _noalloc_raw(b, d1, splits, out_n, lse_n)
        assert st == 0, pa.last_error()
        out_r, lse_r = pa.decode(d2["q"], d2["cache"], d2["table"], d2["seq"], b.max_seq_len,
                                 b.scale, k=d2["k"], v=d2["v"], slot_mapping=d2["slots"],
                                 num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out_n, out_r) and torch.equal(lse_n, lse_r), name
        # raw bits: the pool's unused slots hold NaN
        assert torch.equal(d1["cache"].view(torch.int16), d2["cache"].view(torch.int16))
        cache = O.cache_write_kv(b.cache, b.k_new, b.v_new, b.slot_mapping)
        oref, lref = O.paged_decode(b.q, cache, b.block_table, b.seq_lens, b.scale)
        check_close(to_f64(out_n), oref, f"noalloc {name} out")
        check_lse(lse_n.cpu().numpy().astype(np.float64), lref, f"noalloc {name} lse")
        assert np.array_equal(bits(d1["cache"]), cache)
