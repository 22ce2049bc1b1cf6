"""The C ABI on the host: the library loads, exports every symbol include/pa.h
declares, its integer helpers match the oracle bit for bit, and argument
validation rejects bad calls before anything reaches the GPU (no compute calls
here; these run without a GPU)."""
import ctypes as C
import os
import re

import pytest

import oracle.pa_oracle as O
import paged_kv_attention_pa_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.library_path()):
        pytest.fail("libpa.so is not built: run `python -m paged_kv_attention_pa_amd.build`")
    return pa.library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_operations():
    names = _declared()
    for op in ("pa_cache_write", "pa_decode", "pa_prefill_varlen", "pa_mla_decode", "pa_lse_merge"):
        assert op in names


def test_library_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(pa.EXPORTED_SYMBOLS), (names, pa.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n
    # the exports are C symbols (no C++ mangling)
    out = os.popen(f"nm -D --defined-only {pa.library_path()}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


@pytest.mark.parametrize("max_len", [0, 1, 16, 511, 512, 513, 4096, 8190, 8192, 131072, 10 ** 6])
@pytest.mark.parametrize("cus", [1, 2, 80, 256, 304])
def test_num_kv_splits_matches_oracle(lib, max_len, cus):
    assert pa.num_kv_splits(max_len, cus) == O.num_kv_splits(max_len, cus)


def test_long_context_split_count(lib):
    # 131072 keys on 256 compute units: 256 splits (cap 512 not reached)
    assert pa.num_kv_splits(131072, 256) == 256


def test_workspace_bytes(lib):
    assert pa.decode_workspace_bytes(64, 32, 128, 16) == 64 * 32 * 16 * 129 * 4
    assert pa.decode_workspace_bytes(4, 64, 128, 256) == 4 * 64 * 256 * 129 * 4
    assert pa.decode_workspace_bytes(-1, 32, 128, 16) == 0


def test_decode_workspace_size_queries(lib):
    """The size queries return what pa_decode / pa_mla_decode check for, for
    explicit split counts (the automatic count needs a device)."""
    sz = C.c_size_t(0)
    # 64 requests, 32 q heads, 4 splits over 8192 keys: the split partials
    assert lib.pa_decode_workspace_size(1, 64, 8192, 16, 32, 8, 128, 4, 0, C.byref(sz)) == 0
    assert sz.value == 64 * 32 * 4 * 129 * 4
    # one split covers everything: no workspace, unless only partials are wanted
    assert lib.pa_decode_workspace_size(1, 64, 8192, 16, 32, 8, 128, 1, 0, C.byref(sz)) == 0
    assert sz.value == 0
    assert lib.pa_decode_workspace_size(1, 64, 8192, 16, 32, 8, 128, 1, 1, C.byref(sz)) == 0
    assert sz.value == 64 * 32 * 1 * 129 * 4
    # 16 splits of a 300-key batch: pages of 16 -> P = 32, ten splits hold keys
    assert lib.pa_decode_workspace_size(0, 3, 300, 16, 8, 2, 128, 16, 0, C.byref(sz)) == 0
    assert sz.value == 3 * 8 * 16 * 129 * 4
    assert lib.pa_mla_decode_workspace_size(128, 8192, 64, 128, 512, 3, 0, C.byref(sz)) == 0
    assert sz.value == 128 * 128 * 3 * 513 * 4
    assert lib.pa_mla_decode_workspace_size(128, 64, 64, 128, 512, 2, 0, C.byref(sz)) == 0
    assert sz.value == 0                      # 64 keys fit one page, one split
    for args in [(1, -1, 10, 16, 8, 2, 128, 2, 0), (1, 2, 10, 24, 8, 2, 128, 2, 0),
                 (1, 2, 10, 16, 0, 2, 128, 2, 0), (1, 2, 10, 16, 8, 2, 128, -1, 0)]:
        assert lib.pa_decode_workspace_size(*args, C.byref(sz)) == INVALID, args
        assert pa.last_error() != ""
    assert lib.pa_decode_workspace_size(1, 2, 10, 16, 8, 2, 128, 2, 0, None) == INVALID
    assert lib.pa_mla_decode_workspace_size(2, 10, 8, 16, 512, 2, 0, C.byref(sz)) == INVALID


@pytest.mark.parametrize("B,hkv,L,cus,want", [
    (64, 8, 8192, 256, 16),       # 512 pairs already fill 256 CUs twice: the pages' count
    (3, 2, 4096, 256, 64),        # 6 pairs: raised to 64 splits of 64 keys
    (1, 8, 4096, 256, 64),        # 8 pairs: ceil(512 / 8) = 64, also the 64-key floor
    (4, 8, 131072, 256, 256),     # the pages' count is already 256
    (2, 1, 100000, 256, 256),     # 2 pairs want 256 splits, below the 2 x CUs cap
    (1, 1, 100000, 256, 512),     # one pair: capped at 2 x CUs
    (3, 2, 512, 256, 1),          # the pages' rule does not split: one pass stays
    (3, 2, 600, 256, 10),         # 2 by the rule, raised to ceil(600 / 64) = 10
    (0, 0, 4096, 0, 2),           # non-positive counts read as 1: capped at 2 x 1 CU
])
def test_decode_split_helper(lib, B, hkv, L, cus, want):
    n = pa.decode_num_kv_splits(B, hkv, L, cus)
    assert n == want
    assert n >= O.num_kv_splits(L, max(cus, 1))


def test_mla_split_helper(lib):
    for B, L, cus in [(128, 8192, 256), (1, 8192, 256), (4, 100, 256), (300, 1000, 256)]:
        n = pa.mla_num_kv_splits(B, L, cus)
        assert 1 <= n <= max(1, pa.num_kv_splits(L, cus))
        assert n <= max(1, -(-L // 64))


def _null():
    return None


def _decode(lib, **kw):
    args = dict(dtype=1, q=1 << 20, k=None, v=None, cache=1 << 21, nb=100, bs=16, table=1 << 22,
                maxb=64, slots=None, seq=1 << 23, B=4, maxlen=1000, hq=32, hkv=8, d=128,
                scale=0.1, splits=1, ws=None, wsb=0, out=1 << 24, lse=None)
    args.update(kw)
    a = args
    return lib.pa_decode(a["dtype"], a["q"], a["k"], a["v"], a["cache"], a["nb"], a["bs"],
                         a["table"], a["maxb"], a["slots"], a["seq"], a["B"], a["maxlen"],
                         a["hq"], a["hkv"], a["d"], a["scale"], a["splits"], a["ws"], a["wsb"],
                         a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(bs=8), INVALID),                  # block size not a multiple of 16
    (dict(bs=0), INVALID),
    (dict(hq=30, hkv=8), INVALID),          # Hq % Hkv != 0
    (dict(d=96), UNSUPPORTED),              # head_dim outside this build
    (dict(d=100), INVALID),                 # not a multiple of 8
    (dict(hq=96, hkv=8), UNSUPPORTED),      # group 12
    (dict(q=None), INVALID),
    (dict(out=None), WORKSPACE),            # partial-only mode needs a workspace
    (dict(out=None, lse=1 << 29), INVALID), # lse requested without out
    (dict(table=None), INVALID),
    (dict(k=1 << 25), INVALID),             # k without v / slots
    (dict(k=1 << 25, v=1 << 26), INVALID),  # k, v without slots
    (dict(slots=1 << 27), INVALID),         # slots without k, v
    (dict(maxlen=2000, maxb=64), INVALID),  # longer than the table can address
    (dict(dtype=7), INVALID),
    (dict(splits=-1), INVALID),
    (dict(splits=4, ws=None), WORKSPACE),   # split path needs a workspace
    (dict(splits=4, ws=1 << 28, wsb=100), WORKSPACE),
])
def test_decode_validation(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert pa.last_error() != ""


def test_decode_empty_batch_is_noop(lib):
    assert _decode(lib, B=0, q=None, out=None) == 0
    assert pa.last_error() == ""


def test_cache_write_validation(lib):
    f = lib.pa_cache_write
    assert f(0, 1, 1, 1024, 2, 1024, 3, 10, 16, 8, 128, 4, 0, None) == 0     # zero tokens
    assert f(0, 1, 1, 1024, 2, 1024, 3, 10, 12, 8, 128, 4, 5, None) == INVALID  # block 12
    assert f(0, 1, None, 1024, 2, 1024, 3, 10, 16, 8, 128, 4, 5, None) == INVALID
    assert f(0, 1, 1, 100, 2, 1024, 3, 10, 16, 8, 128, 4, 5, None) == INVALID  # short stride
    assert f(1, 0, 1, 512, 2, 64, 3, 10, 64, 1, 576, 4, 5, None) == UNSUPPORTED  # MLA fp32
    assert f(1, 1, 1, 512, 2, 64, 3, 10, 64, 2, 576, 4, 5, None) == INVALID  # MLA 2 heads
    assert f(9, 1, 1, 512, 2, 64, 3, 10, 64, 1, 576, 4, 5, None) == INVALID  # bad layout


def test_prefill_validation(lib):
    f = lib.pa_prefill_varlen
    base = [1, 1, None, None, 2, 100, 16, 3, 64, None, 4, 5, 2, 100, 50, 300,
            32, 8, 128, 0.1, 1, 6, None, None]
    bad = list(base); bad[0] = 0                   # fp32 prefill
    assert f(*bad) == UNSUPPORTED
    bad = list(base); bad[20] = 2                  # causal flag
    assert f(*bad) == INVALID
    bad = list(base); bad[14] = 200                # max_query_len > num_tokens
    assert f(*bad) == INVALID
    bad = list(base); bad[10] = None               # query_start_loc
    assert f(*bad) == INVALID
    bad = list(base); bad[16] = 20                 # 20 % 8
    assert f(*bad) == INVALID


def test_mla_validation(lib):
    f = lib.pa_mla_decode
    base = [1, 128 * 512, 512, 2, 128 * 64, 64, None, None, 3, 100, 64, 4, 200, None, 5, 8,
            8192, 128, 512, 64, 0.07, 1, None, 0, 6, None, None]
    bad = list(base); bad[18] = 320                # head 320 not built
    assert f(*bad) == UNSUPPORTED
    bad = list(base); bad[17] = 24                 # heads not a multiple of 16
    assert f(*bad) == UNSUPPORTED
    bad = list(base); bad[2] = 100                 # q_nope head stride < 512
    assert f(*bad) == INVALID
    bad = list(base); bad[6] = 7                   # kv_c without k_pe
    assert f(*bad) == INVALID
    bad = list(base); bad[21] = 4                  # split without workspace
    assert f(*bad) == WORKSPACE


def test_lse_merge_validation(lib):
    f = lib.pa_lse_merge
    assert f(1, 4, 8, 0, 128, 1, 2, None, None) == INVALID        # zero splits
    assert f(1, 4, 8, 2, 2048, 1, 2, None, None) == UNSUPPORTED   # Dv too wide
    assert f(None, 4, 8, 2, 128, 1, 2, None, None) == INVALID
    assert f(None, 0, 8, 2, 128, 1, 2, None, None) == 0           # nothing to do


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import paged_kv_attention_pa_amd._binding as b
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "_LIB_PATH", str(tmp_path / "libpa.so"))
    with pytest.raises(pa.PaError):
        b.library()


def test_scale_must_be_finite_non_negative(lib):
    assert _decode(lib, scale=-0.5) == INVALID
    assert _decode(lib, scale=float("inf")) == INVALID
    assert _decode(lib, scale=float("nan")) == INVALID


def test_balanced_helpers(lib):
    # eight waves per compute unit: one range per CU for 8 KV heads, more for fewer
    assert pa.decode_balanced_num_ranges(8, 256) == 256
    assert pa.decode_balanced_num_ranges(2, 256) == 1024
    assert pa.decode_balanced_num_ranges(1, 256) == 2048
    assert pa.decode_balanced_num_ranges(16, 256) == 128
    assert pa.decode_balanced_num_ranges(8, 0) == 1
    # cu[B + 1] rounded to 256 B, then (ranges + B) * H rows of Dv + 4 fp32
    assert pa.decode_balanced_workspace_bytes(64, 32, 128, 256) == 512 + (256 + 64) * 32 * 132 * 4
    assert pa.decode_balanced_workspace_bytes(63, 32, 128, 256) == 256 + (256 + 63) * 32 * 132 * 4
    assert pa.decode_balanced_workspace_bytes(4, 64, 128, 256) == 256 + 260 * 64 * 132 * 4
    assert pa.decode_balanced_workspace_bytes(128, 128, 512, 256) == 768 + 384 * 128 * 516 * 4
    assert pa.decode_balanced_workspace_bytes(-1, 32, 128, 256) == 0
    assert pa.decode_balanced_workspace_bytes(4, 32, 128, 0) == 0


def test_balanced_validation(lib):
    f = lib.pa_decode_balanced
    need = pa.decode_balanced_workspace_bytes(4, 32, 128, 16)
    #        q  cache  nb  bs  table maxb seq B  hq  hkv d    scale nr  ws       wsb   out  lse
    base = [1, 2, 100, 16, 3, 64, 4, 4, 32, 8, 128, 0.1, 16, 1 << 20, need, 5, None, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a12=0) == INVALID                    # no ranges
    assert call(a14=need - 1) == WORKSPACE           # workspace too small
    assert call(a13=None) == WORKSPACE
    assert call(a13=(1 << 20) + 4) == INVALID        # misaligned workspace
    assert call(a10=64) == UNSUPPORTED               # head_dim 64
    assert call(a8=96) == UNSUPPORTED                # group 12
    assert call(a11=-1.0) == INVALID                 # negative scale
    assert call(a3=24) == INVALID                    # block size 24
    assert call(a15=None) == INVALID                 # no output
    assert call(a5=1 << 30, a7=1 << 20) == UNSUPPORTED   # chunk count past int32
    assert call(a8=12, a9=6) == UNSUPPORTED              # 6 KV heads: not whole rows of 1/2/4/8
    m = lib.pa_decode_balanced_merge
    assert m(1 << 20, need - 1, 4, 32, 128, 16, 5, None, None) == WORKSPACE
    assert m(1 << 20, need, 4, 32, 128, 0, 5, None, None) == INVALID
    assert m(1 << 20, need, 4, 32, 64, 16, 5, None, None) == UNSUPPORTED   # head_dim_v 64
    assert m(1 << 20, need, 4, 32, 128, 16, None, None, None) == INVALID
    assert m(None, 0, 0, 32, 128, 16, None, None, None) == WORKSPACE


def test_mla_balanced_validation(lib):
    f = lib.pa_mla_decode_balanced
    need = pa.decode_balanced_workspace_bytes(4, 128, 512, 16)
    base = [1, 128 * 512, 512, 2, 128 * 64, 64, 3, 100, 64, 4, 200, 5, 4, 128, 512, 64, 0.07, 16,
            1 << 20, need, 6, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(17, 0) == INVALID                     # no ranges
    assert call(19, need - 1) == WORKSPACE            # workspace too small
    assert call(14, 320) == UNSUPPORTED               # kv_lora_rank 320
    assert call(13, 24) == UNSUPPORTED                # heads not a multiple of 16
    assert call(2, 100) == INVALID                    # q_nope head stride < 512
    assert call(20, None) == INVALID                  # no output
    assert call(18, (1 << 20) + 8) == INVALID         # misaligned workspace

    def sized(num_seqs, max_blocks):
        a = list(base)
        a[12], a[10] = num_seqs, max_blocks
        return f(*a)

    # the unit list (2 max_blocks chunks + 5 overhead units per request at
    # block 64) must stay below 2^31: 2^20 (2046 + 5) units exceed it, though
    # 2^20 * 2046 chunks alone would not; 2^20 (2040 + 5) fit, and only the
    # workspace is then too small
    assert sized(1 << 20, 1023) == UNSUPPORTED
    assert sized(1 << 20, 1020) == WORKSPACE


def test_fp8_write_validation(lib):
    f = lib.pa_cache_write_fp8
    #     layout k  kst   v  vst   cache nb  bs  hkv d    slots T  ks   vs   stream
    base = [0, 1, 1024, 2, 1024, 3, 10, 16, 8, 128, 4, 5, 0.5, 0.25, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(11, 0) == 0                            # zero tokens: nothing to do
    assert call(12, 0.0) == INVALID                    # k_scale 0
    assert call(13, float("inf")) == INVALID           # v_scale not finite
    assert call(12, float("nan")) == INVALID
    assert call(7, 12) == INVALID                      # block size 12
    assert call(2, 100) == INVALID                     # k stride too short
    assert call(0, 9) == INVALID                       # unknown layout
    assert call(1, None) == INVALID                    # no k
    # MLA layout: one KV head, a rank + 64 row; v_scale unused (zero tokens: no launch)
    assert f(1, 1, 512, 2, 64, 3, 10, 64, 1, 576, 4, 0, 0.5, 0.0, None) == 0
    assert f(1, 1, 512, 2, 64, 3, 10, 64, 2, 576, 4, 5, 0.5, 1.0, None) == INVALID


def test_fp8_decode_validation(lib):
    f = lib.pa_decode_fp8
    need = pa.decode_balanced_workspace_bytes(4, 32, 128, 16)
    #       q  k     v     cache nb  bs  table maxb slots seq B  hq  hkv d    sc   ks   vs  nr
    base = [1, None, None, 2, 100, 16, 3, 64, None, 4, 4, 32, 8, 128, 0.1, 0.5, 0.5, 16,
            1 << 20, need, 5, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(15, 0.0) == INVALID                    # k_scale
    assert call(16, -1.0) == INVALID                   # v_scale
    assert call(13, 64) == UNSUPPORTED                 # head_dim 64
    assert call(11, 96) == UNSUPPORTED                 # group 12
    six = list(base)
    six[11], six[12] = 12, 6                           # 6 KV heads: not whole rows of 1/2/4/8
    assert f(*six) == UNSUPPORTED
    assert call(19, need - 1) == WORKSPACE
    assert call(18, (1 << 20) + 4) == INVALID          # misaligned workspace
    assert call(1, 7) == INVALID                       # k without v
    assert call(17, -1) == INVALID                     # negative range count
    assert call(10, 0) == 0                            # empty batch


def test_fp8_prefill_validation(lib):
    f = lib.pa_prefill_varlen_fp8
    #       q  k     v     cache nb  bs  table maxb slots qsl seq N  T    maxq maxs hq hkv d
    base = [1, None, None, 2, 100, 16, 3, 64, None, 4, 5, 2, 100, 50, 300, 32, 8, 128,
            0.1, 0.5, 0.5, 1, 6, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(19, 0.0) == INVALID                    # k_scale
    assert call(20, float("nan")) == INVALID           # v_scale
    assert call(21, 2) == INVALID                      # causal flag
    assert call(13, 200) == INVALID                    # max_query_len > num_tokens
    assert call(17, 64) == UNSUPPORTED                 # head_dim 64
    assert call(9, None) == INVALID                    # query_start_loc
    assert call(11, 0) == 0                            # no requests


def test_fp8_mla_validation(lib):
    f = lib.pa_mla_decode_fp8
    need = pa.decode_balanced_workspace_bytes(4, 128, 512, 16)
    base = [1, 128 * 512, 512, 2, 128 * 64, 64, None, None, 3, 100, 64, 4, 64, None, 5, 4, 128, 512,
            64, 0.07, 0.5, 16, 1 << 20, need, 6, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(20, 0.0) == INVALID                    # kv_scale
    assert call(17, 256) == UNSUPPORTED                # rank 256 is bf16 only
    assert call(23, need - 1) == WORKSPACE
    assert call(6, 9) == INVALID                       # kv_c without k_pe
    assert call(21, -2) == INVALID                     # negative range count


def test_mla_prefill_validation(lib):
    f = lib.pa_mla_prefill
    need = pa.mla_prefill_workspace_bytes(2, 700, 16)
    up = lambda x: (x + 255) // 256 * 256
    # key offsets + list length, work list (2 + 700 // 128 + 1 entries of 8 B),
    # projected keys, projected values
    assert need == up(4 * 4) + up(8 * 8) + up(700 * 16 * 192 * 2) + up(700 * 16 * 128 * 2)
    #       q  qst       qsh  kv_c  k_pe  cache nb  bs  table maxb slots qsl seq N  T    maxq keys
    base = [1, 16 * 192, 192, None, None, 2, 100, 64, 3, 64, None, 4, 5, 2, 300, 200, 700,
            7, 16, 512, 64, 128, 128, 0.07, 1 << 20, need, 6, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(19, 256) == UNSUPPORTED                # kv_lora_rank 256
    assert call(21, 192) == UNSUPPORTED                # qk_nope 192
    assert call(25, need - 1) == WORKSPACE
    assert call(24, (1 << 20) + 16) == INVALID         # misaligned workspace
    assert call(2, 100) == INVALID                     # head stride < 192
    assert call(15, 400) == INVALID                    # max_query_len > num_tokens
    assert call(3, 9) == INVALID                       # kv_c without k_pe
    assert call(17, None) == INVALID                   # no weight
    assert call(23, -1.0) == INVALID                   # negative scale
    assert call(13, 0) == 0                            # no requests
