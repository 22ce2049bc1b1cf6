"""ctypes marshalling for libpa.so: tensors -> device pointers, shapes -> ints.

No computation happens here.  Output buffers and workspaces are allocated
with torch when the caller does not pass them (that is memory plumbing; the
C ABI itself never allocates).
"""

from __future__ import annotations

import ctypes as C
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libpa.so")

PA_F32, PA_BF16 = 0, 1
PA_LAYOUT_KV, PA_LAYOUT_MLA = 0, 1
_STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID", 2: "PA_ERR_UNSUPPORTED",
           3: "PA_ERR_WORKSPACE", 4: "PA_ERR_HIP"}

# every symbol include/pa.h declares, with (restype, argtypes)
_vp, _i32, _i64, _f32, _sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
_SIGNATURES = {
    "pa_num_kv_splits": (_i32, [_i32, _i32]),
    "pa_decode_num_kv_splits": (_i32, [_i32, _i32, _i32, _i32]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "pa_mla_num_kv_splits": (_i32, [_i32, _i32, _i32]),
    "pa_device_num_cus": (_i32, []),
    "pa_decode_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                        C.POINTER(_sz)]),
    "pa_mla_decode_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                            C.POINTER(_sz)]),
    "pa_last_error": (C.c_char_p, []),
    "pa_cache_write": (_i32, [_i32, _i32, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32,
                              _vp, _i32, _vp]),
    "pa_decode": (_i32, [_i32, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i32, _i32,
                         _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp, _vp, _vp]),
    "pa_prefill_varlen": (_i32, [_i32, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _vp,
                                 _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp,
                                 _vp]),
    "pa_mla_decode": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp,
                             _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                             _vp, _vp, _vp]),
    "pa_lse_merge": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "pa_decode_balanced_num_ranges": (_i32, [_i32, _i32]),
    "pa_decode_balanced_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "pa_decode_balanced": (_i32, [_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                  _f32, _i32, _vp, _sz, _vp, _vp, _vp]),
    "pa_decode_balanced_merge": (_i32, [_vp, _sz, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "pa_mla_decode_balanced": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i32, _vp,
                                      _i32, _vp, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                      _vp, _vp, _vp]),
    "pa_plan_mixed": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_mixed_attention": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _f32,
                                  _vp, _sz, _vp, _vp, _vp]),
    "pa_plan_cascade": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_cache_write_fp8": (_i32, [_i32, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp,
                                  _i32, _f32, _f32, _vp]),
    "pa_mla_decode_fp8": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp,
                                 _i32, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _f32, _i32, _vp,
                                 _sz, _vp, _vp, _vp]),
    "pa_mla_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "pa_mla_prefill": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _vp,
                              _i32, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                              _sz, _vp, _vp, _vp]),
    "pa_prefill_varlen_fp8": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _vp,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _f32, _f32,
                                     _i32, _vp, _vp, _vp]),
    "pa_decode_fp8": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i32, _i32,
                             _i32, _i32, _f32, _f32, _f32, _i32, _vp, _sz, _vp, _vp, _vp]),
    "pa_cascade_attention": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp,
                                    _f32, _vp, _sz, _vp, _vp, _vp]),
    "pa_decode_noalloc": (_i32, [_i32, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i32,
                                 _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lock = threading.Lock()
_lib = None


class PaError(RuntimeError):
    """A non-OK status from libpa.so (or the library is missing)."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library() -> C.CDLL:
    """Load libpa.so (once).  Raises PaError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise PaError(-1, f"{_LIB_PATH} is missing; build it with "
                                  "`python -m paged_kv_attention_pa_amd.build`")
            lib = C.CDLL(_LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def last_error() -> str:
    return library().pa_last_error().decode()


def _check(status: int):
    if status != 0:
        raise PaError(status, last_error())


# ------------------------------------------------------------------ helpers
def num_kv_splits(max_seq_len: int, num_cus: int) -> int:
    return library().pa_num_kv_splits(int(max_seq_len), int(num_cus))


def decode_num_kv_splits(num_seqs: int, num_kv_heads: int, max_seq_len: int, num_cus: int) -> int:
    return library().pa_decode_num_kv_splits(int(num_seqs), int(num_kv_heads), int(max_seq_len),
                                             int(num_cus))


def mla_num_kv_splits(num_seqs: int, max_seq_len: int, num_cus: int) -> int:
    return library().pa_mla_num_kv_splits(int(num_seqs), int(max_seq_len), int(num_cus))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim_v: int, num_splits: int) -> int:
    return library().pa_decode_workspace_bytes(int(num_seqs), int(num_q_heads), int(head_dim_v),
                                               int(num_splits))


def decode_workspace_size(dtype: int, num_seqs: int, max_seq_len: int, block_size: int,
                          num_q_heads: int, num_kv_heads: int, head_dim: int, num_splits: int,
                          partials_only: bool = False) -> int:
    """Bytes of workspace ``pa_decode`` needs for these sizes (0 = none)."""
    n = C.c_size_t(0)
    _check(library().pa_decode_workspace_size(int(dtype), int(num_seqs), int(max_seq_len),
                                              int(block_size), int(num_q_heads),
                                              int(num_kv_heads), int(head_dim), int(num_splits),
                                              1 if partials_only else 0, C.byref(n)))
    return n.value


def mla_decode_workspace_size(num_seqs: int, max_seq_len: int, block_size: int, num_heads: int,
                              kv_lora_rank: int, num_splits: int,
                              partials_only: bool = False) -> int:
    """Bytes of workspace ``pa_mla_decode`` needs for these sizes (0 = none)."""
    n = C.c_size_t(0)
    _check(library().pa_mla_decode_workspace_size(int(num_seqs), int(max_seq_len),
                                                  int(block_size), int(num_heads),
                                                  int(kv_lora_rank), int(num_splits),
                                                  1 if partials_only else 0, C.byref(n)))
    return n.value


def decode_balanced_num_ranges(num_kv_heads: int, num_cus: int) -> int:
    return library().pa_decode_balanced_num_ranges(int(num_kv_heads), int(num_cus))


def decode_balanced_workspace_bytes(num_seqs: int, num_heads: int, head_dim_v: int,
                                    num_ranges: int) -> int:
    return library().pa_decode_balanced_workspace_bytes(int(num_seqs), int(num_heads),
                                                        int(head_dim_v), int(num_ranges))


def device_num_cus() -> int:
    return library().pa_device_num_cus()


class MixedPlan(C.Structure):
    """pa_mixed_plan_t: the split of a mixed batch into its leading decode
    requests and the prefill rest, with the decode group's schedule."""

    _fields_ = [(n, C.c_int) for n in (
        "num_seqs", "num_tokens", "num_decode", "max_decode_seq_len", "prefill_tokens",
        "max_query_len", "max_seq_len", "num_q_heads", "num_kv_heads", "head_dim",
        "block_size", "max_blocks_per_seq", "decode_ranges", "decode_splits")] + [
        ("workspace_bytes", C.c_size_t)]

    def __repr__(self):
        return "MixedPlan(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class CascadePlan(C.Structure):
    """pa_cascade_plan_t: the mixed-batch plan of the suffixes plus the shared
    prefix's key ranges."""

    _fields_ = [("suffix", MixedPlan), ("prefix_blocks", C.c_int), ("prefix_len", C.c_int),
                ("prefix_splits", C.c_int), ("split_keys", C.c_int),
                ("workspace_bytes", C.c_size_t)]

    def __repr__(self):
        return (f"CascadePlan(prefix_blocks={self.prefix_blocks}, prefix_len={self.prefix_len}, "
                f"prefix_splits={self.prefix_splits}, split_keys={self.split_keys}, "
                f"workspace_bytes={self.workspace_bytes}, suffix={self.suffix!r})")


def _host_i32(x, name):
    """A host int32 ctypes array from a list, numpy array or CPU tensor."""
    if hasattr(x, "is_cuda"):
        _need(not x.is_cuda, f"{name}: pa_plan_mixed reads host copies (got a GPU tensor)")
        x = x.tolist()
    vals = [int(t) for t in x]
    return (C.c_int32 * max(len(vals), 1))(*vals), len(vals)


def plan_mixed(query_start_loc, seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
               block_size: int, max_blocks_per_seq: int, num_cus: int = 0) -> MixedPlan:
    """Host-only plan of a mixed batch (pa_plan_mixed) from host copies of
    query_start_loc [N + 1] and seq_lens [N]."""
    qsl, nq = _host_i32(query_start_loc, "query_start_loc")
    sl, n = _host_i32(seq_lens, "seq_lens")
    _need(nq == n + 1, "query_start_loc must have num_seqs + 1 entries")
    plan = MixedPlan()
    _check(library().pa_plan_mixed(qsl, sl, n, int(num_q_heads), int(num_kv_heads),
                                   int(head_dim), int(block_size), int(max_blocks_per_seq),
                                   int(num_cus), C.byref(plan)))
    return plan


def plan_cascade(query_start_loc, seq_lens, num_common_prefix_blocks: int, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, block_size: int, max_blocks_per_seq: int,
                 num_cus: int = 0) -> CascadePlan:
    """Host-only plan of a batch whose block-table rows share their first
    num_common_prefix_blocks pages (pa_plan_cascade)."""
    qsl, nq = _host_i32(query_start_loc, "query_start_loc")
    sl, n = _host_i32(seq_lens, "seq_lens")
    _need(nq == n + 1, "query_start_loc must have num_seqs + 1 entries")
    plan = CascadePlan()
    _check(library().pa_plan_cascade(qsl, sl, n, int(num_common_prefix_blocks), int(num_q_heads),
                                     int(num_kv_heads), int(head_dim), int(block_size),
                                     int(max_blocks_per_seq), int(num_cus), C.byref(plan)))
    return plan


# ------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    for t in ts:
        if t is not None:
            _need(t.is_cuda, "every tensor must be on the GPU")
            _need(t.is_contiguous(), "tensors must be contiguous")


def _int_tensor(t, dtype, name):
    torch = _torch()
    _need(t.dtype == getattr(torch, dtype), f"{name} must be {dtype}")


# ------------------------------------------------------------- entry points
def cache_write(kv_cache, k, v, slot_mapping, layout: int = PA_LAYOUT_KV, stream=None):
    """Store new rows at slot_mapping.  GQA: k, v [T, Hkv, D] into
    kv_cache [nb, 2, bs, Hkv, D].  MLA: k = kv_c [T, R], v = k_pe [T, 64]
    into kv_cache [nb, bs, R + 64]."""
    _dev(kv_cache, k, v, slot_mapping)
    _int_tensor(slot_mapping, "int64", "slot_mapping")
    dt = _dtype_code(kv_cache)
    _need(k.dtype == kv_cache.dtype and v.dtype == kv_cache.dtype, "k/v dtype must match the cache")
    T = k.shape[0]
    if layout == PA_LAYOUT_KV:
        nb, _, bs, hkv, d = kv_cache.shape
        _need(tuple(k.shape) == (T, hkv, d) and tuple(v.shape) == (T, hkv, d), "k/v shape mismatch")
        ks = vs = hkv * d
    else:
        nb, bs, row = kv_cache.shape
        hkv, d = 1, row
        ks, vs = k.shape[1], v.shape[1]
        _need(ks + vs == row, "kv_c/k_pe widths must add up to the cache row")
    _need(slot_mapping.numel() == T, "slot_mapping must have one entry per token")
    _check(library().pa_cache_write(layout, dt, _ptr(k), ks, _ptr(v), vs, _ptr(kv_cache), nb, bs,
                                    hkv, d, _ptr(slot_mapping), T, _stream(stream)))


def _fp8_cache(kv_cache):
    torch = _torch()
    _need(kv_cache.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)),
          "an FP8 cache is uint8 (or float8_e4m3fn) storage")


def cache_write_fp8(kv_cache, k, v, slot_mapping, k_scale: float, v_scale: float = 1.0,
                    layout: int = PA_LAYOUT_KV, stream=None):
    """Quantise bf16 rows to E4M3 (x / scale) and store them at slot_mapping.
    GQA: k, v [T, Hkv, D] into kv_cache [nb, 2, bs, Hkv, D] uint8.  MLA: k =
    kv_c [T, R], v = k_pe [T, 64] into kv_cache [nb, bs, R + 64] uint8, the
    row with k_scale."""
    torch = _torch()
    _dev(kv_cache, k, v, slot_mapping)
    _fp8_cache(kv_cache)
    _int_tensor(slot_mapping, "int64", "slot_mapping")
    _need(k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16, "k/v must be bf16")
    T = k.shape[0]
    if layout == PA_LAYOUT_KV:
        nb, _, bs, hkv, d = kv_cache.shape
        _need(tuple(k.shape) == (T, hkv, d) and tuple(v.shape) == (T, hkv, d), "k/v shape mismatch")
        ks = vs = hkv * d
    else:
        nb, bs, row = kv_cache.shape
        hkv, d = 1, row
        ks, vs = k.shape[1], v.shape[1]
        _need(ks + vs == row, "kv_c/k_pe widths must add up to the cache row")
    _need(slot_mapping.numel() == T, "slot_mapping must have one entry per token")
    _check(library().pa_cache_write_fp8(layout, _ptr(k), ks, _ptr(v), vs, _ptr(kv_cache), nb, bs,
                                        hkv, d, _ptr(slot_mapping), T, float(k_scale),
                                        float(v_scale), _stream(stream)))


def decode_fp8(q, kv_cache, block_table, seq_lens, scale: float, k_scale: float, v_scale: float,
               k=None, v=None, slot_mapping=None, num_ranges: int = 0, workspace=None, out=None,
               lse=None, return_lse: bool = True, stream=None):
    """GQA decode over an FP8 (E4M3) cache [nb, 2, bs, Hkv, D] uint8 with
    per-tensor k_scale / v_scale; q bf16 [B, Hq, D].  Token-balanced schedule
    (num_ranges = 0: one range per CU for 8 KV heads).  Returns (out, lse)."""
    torch = _torch()
    _dev(q, kv_cache, block_table, seq_lens, k, v, slot_mapping, workspace, out, lse)
    _fp8_cache(kv_cache)
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    _need(q.dtype == torch.bfloat16, "q must be bf16")
    B, Hq, D = q.shape
    nb, _, bs, hkv, d2 = kv_cache.shape
    _need(d2 == D, "head_dim mismatch")
    nr = int(num_ranges) or decode_balanced_num_ranges(hkv, device_num_cus())
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = decode_balanced_workspace_bytes(B, Hq, D, nr)
        workspace = torch.empty(max(1, need // 4), dtype=torch.float32, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(library().pa_decode_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), nb, bs,
                                   _ptr(block_table), block_table.shape[1], _ptr(slot_mapping),
                                   _ptr(seq_lens), B, Hq, hkv, D, float(scale), float(k_scale),
                                   float(v_scale), nr, _ptr(workspace), wbytes, _ptr(out),
                                   _ptr(lse), _stream(stream)))
    return out, lse


def prefill_varlen_fp8(q, kv_cache, block_table, query_start_loc, seq_lens, max_query_len: int,
                       max_seq_len: int, scale: float, k_scale: float, v_scale: float, k=None,
                       v=None, slot_mapping=None, causal: bool = True, out=None, lse=None,
                       return_lse: bool = True, stream=None):
    """Varlen (chunked) prefill over an FP8 (E4M3) cache [nb, 2, bs, Hkv, D]
    uint8; q [T, Hq, D] bf16.  Returns (out [T, Hq, D], lse [T, Hq])."""
    torch = _torch()
    _dev(q, kv_cache, block_table, query_start_loc, seq_lens, k, v, slot_mapping, out, lse)
    _fp8_cache(kv_cache)
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    _int_tensor(query_start_loc, "int32", "query_start_loc")
    _need(q.dtype == torch.bfloat16, "q must be bf16")
    T, Hq, D = q.shape
    nb, _, bs, hkv, _ = kv_cache.shape
    N = seq_lens.numel()
    _need(query_start_loc.numel() == N + 1, "query_start_loc must have num_seqs + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _check(library().pa_prefill_varlen_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), nb, bs,
                                           _ptr(block_table), block_table.shape[1],
                                           _ptr(slot_mapping), _ptr(query_start_loc),
                                           _ptr(seq_lens), N, T, int(max_query_len),
                                           int(max_seq_len), Hq, hkv, D, float(scale),
                                           float(k_scale), float(v_scale), 1 if causal else 0,
                                           _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def decode(q, kv_cache, block_table, seq_lens, max_seq_len: int, scale: float,
           k=None, v=None, slot_mapping=None, num_splits: int = 0, workspace=None,
           out=None, lse=None, return_lse: bool = True, stage1_only: bool = False,
           stream=None):
    """GQA decode: q [B, Hq, D]; kv_cache [nb, 2, bs, Hkv, D]; returns (out, lse).

    stage1_only: run only the split kernel and return the partials
    [B, Hq, n, D + 1] (a view of the workspace) for ``lse_merge``."""
    torch = _torch()
    _dev(q, kv_cache, block_table, seq_lens, k, v, slot_mapping, workspace, out, lse)
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    dt = _dtype_code(q)
    _need(kv_cache.dtype == q.dtype, "q and cache dtypes must match")
    B, Hq, D = q.shape
    nb, _, bs, hkv, d2 = kv_cache.shape
    _need(d2 == D, "head_dim mismatch")
    if stage1_only:
        out = lse = None
    else:
        if out is None:
            out = torch.empty_like(q)
        if lse is None and return_lse:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = decode_workspace_size(dt, B, max_seq_len, bs, Hq, hkv, D, num_splits, stage1_only)
    if workspace is None and need:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_decode(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), nb, bs,
                               _ptr(block_table), block_table.shape[1], _ptr(slot_mapping),
                               _ptr(seq_lens), B, int(max_seq_len), Hq, hkv, D, float(scale),
                               int(num_splits), _ptr(workspace), wbytes, _ptr(out), _ptr(lse),
                               _stream(stream)))
    if stage1_only:
        n = need // max(1, 4 * B * Hq * (D + 1))    # the split count the call used
        if workspace is None:
            return torch.empty((B, Hq, 0, D + 1), dtype=torch.float32, device=q.device)
        return workspace[: B * Hq * n * (D + 1)].view(B, Hq, n, D + 1)
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024   # PA_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q, kv_cache, block_table, seq_lens, max_seq_len: int, scale: float,
                   k=None, v=None, slot_mapping=None, num_splits: int = 0, out=None, lse=None,
                   return_lse: bool = True, stream=None):
    """``pa_decode_noalloc``: GQA decode whose partials live in the library's
    own device array (no workspace argument).  Returns (out, lse)."""
    torch = _torch()
    _dev(q, kv_cache, block_table, seq_lens, k, v, slot_mapping, out, lse)
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    nb, _, bs, hkv, _ = kv_cache.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(library().pa_decode_noalloc(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), nb, bs,
                                       _ptr(block_table), block_table.shape[1], _ptr(slot_mapping),
                                       _ptr(seq_lens), B, int(max_seq_len), Hq, hkv, D,
                                       float(scale), int(num_splits), _ptr(out), _ptr(lse),
                                       _stream(stream)))
    return out, lse


def decode_balanced(q, kv_cache, block_table, seq_lens, scale: float, num_ranges: int = 0,
                    workspace=None, out=None, lse=None, return_lse: bool = True,
                    merge: bool = True, stream=None):
    """Token-balanced GQA decode (bf16): q [B, Hq, D]; kv_cache [nb, 2, bs, Hkv, D].

    num_ranges = 0 takes ``decode_balanced_num_ranges(Hkv, device_num_cus())``.
    merge=False runs only the first kernel: out / lse then hold just the
    requests that lie inside one range, and the workspace the partials that
    ``decode_balanced_merge`` combines.  Returns (out, lse, workspace, num_ranges)."""
    torch = _torch()
    _dev(q, kv_cache, block_table, seq_lens, workspace, out, lse)
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    _need(q.dtype == torch.bfloat16 and kv_cache.dtype == torch.bfloat16, "bf16 q and cache")
    B, Hq, D = q.shape
    nb, _, bs, hkv, d2 = kv_cache.shape
    _need(d2 == D, "head_dim mismatch")
    nr = int(num_ranges) or decode_balanced_num_ranges(hkv, device_num_cus())
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = decode_balanced_workspace_bytes(B, Hq, D, nr)
    if workspace is None:
        workspace = torch.empty(max(1, need // 4), dtype=torch.float32, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    lib = library()
    _check(lib.pa_decode_balanced(_ptr(q), _ptr(kv_cache), nb, bs, _ptr(block_table),
                                  block_table.shape[1], _ptr(seq_lens), B, Hq, hkv, D,
                                  float(scale), nr, _ptr(workspace), wbytes, _ptr(out),
                                  _ptr(lse), _stream(stream)))
    if merge:
        decode_balanced_merge(workspace, B, Hq, D, nr, out, lse, stream=stream)
    return out, lse, workspace, nr


def decode_balanced_merge(workspace, num_seqs: int, num_heads: int, head_dim_v: int,
                          num_ranges: int, out, lse=None, stream=None):
    """Second kernel of the balanced GQA (head_dim_v 128) or MLA (512 / 256) decode:
    combine the partials of requests that cross ranges into out / lse."""
    _dev(workspace, out, lse)
    wbytes = workspace.numel() * workspace.element_size()
    _check(library().pa_decode_balanced_merge(_ptr(workspace), wbytes, int(num_seqs),
                                              int(num_heads), int(head_dim_v), int(num_ranges),
                                              _ptr(out), _ptr(lse), _stream(stream)))


def prefill_varlen(q, kv_cache, block_table, query_start_loc, seq_lens, max_query_len: int,
                   max_seq_len: int, scale: float, k=None, v=None, slot_mapping=None,
                   causal: bool = True, out=None, lse=None, return_lse: bool = True,
                   stream=None):
    """Varlen (chunked) prefill: q [T, Hq, D]; returns (out [T, Hq, D], lse [T, Hq])."""
    torch = _torch()
    _dev(q, kv_cache, block_table, query_start_loc, seq_lens, k, v, slot_mapping, out, lse)
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    _int_tensor(query_start_loc, "int32", "query_start_loc")
    dt = _dtype_code(q)
    T, Hq, D = q.shape
    nb, _, bs, hkv, _ = kv_cache.shape
    N = seq_lens.numel()
    _need(query_start_loc.numel() == N + 1, "query_start_loc must have num_seqs + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _check(library().pa_prefill_varlen(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), nb, bs,
                                       _ptr(block_table), block_table.shape[1], _ptr(slot_mapping),
                                       _ptr(query_start_loc), _ptr(seq_lens), N, T,
                                       int(max_query_len), int(max_seq_len), Hq, hkv, D,
                                       float(scale), 1 if causal else 0, _ptr(out), _ptr(lse),
                                       _stream(stream)))
    return out, lse


def mixed_attention(plan: MixedPlan, q, kv_cache, block_table, query_start_loc, seq_lens,
                    scale: float, k=None, v=None, slot_mapping=None, workspace=None, out=None,
                    lse=None, return_lse: bool = True, stream=None):
    """One layer of a planned mixed batch (pa_mixed_attention): q [T, Hq, D]
    with the plan's decode requests first; returns (out [T, Hq, D], lse [T, Hq])."""
    return _planned_call(library().pa_mixed_attention, plan, plan, q, kv_cache, block_table,
                         query_start_loc, seq_lens, scale, k, v, slot_mapping, workspace, out,
                         lse, return_lse, stream)


def _planned_call(fn, plan, mp, q, kv_cache, block_table, query_start_loc, seq_lens, scale,
                  k, v, slot_mapping, workspace, out, lse, return_lse, stream):
    torch = _torch()
    _dev(q, kv_cache, block_table, query_start_loc, seq_lens, k, v, slot_mapping, workspace,
         out, lse)
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    _int_tensor(query_start_loc, "int32", "query_start_loc")
    T, Hq, D = q.shape
    nb, _, bs, hkv, _ = kv_cache.shape
    _need(T == mp.num_tokens and seq_lens.numel() == mp.num_seqs and
          query_start_loc.numel() == mp.num_seqs + 1, "tensors do not match the plan's batch")
    _need(Hq == mp.num_q_heads and hkv == mp.num_kv_heads and D == mp.head_dim and
          bs == mp.block_size and block_table.shape[1] == mp.max_blocks_per_seq,
          "tensor shapes do not match the plan")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    if workspace is None and plan.workspace_bytes:
        workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(C.byref(plan), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), nb,
              _ptr(block_table), _ptr(slot_mapping), _ptr(query_start_loc), _ptr(seq_lens),
              float(scale), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def cascade_attention(plan: CascadePlan, q, kv_cache, block_table, query_start_loc, seq_lens,
                      scale: float, k=None, v=None, slot_mapping=None, workspace=None, out=None,
                      lse=None, return_lse: bool = True, stream=None):
    """One layer of a planned shared-prefix batch (pa_cascade_attention);
    returns (out [T, Hq, D], lse [T, Hq])."""
    return _planned_call(library().pa_cascade_attention, plan, plan.suffix, q, kv_cache,
                         block_table, query_start_loc, seq_lens, scale, k, v, slot_mapping,
                         workspace, out, lse, return_lse, stream)


def mla_decode(q_nope, q_pe, kv_cache, block_table, seq_lens, max_seq_len: int, scale: float,
               kv_c=None, k_pe=None, slot_mapping=None, num_splits: int = 0, workspace=None,
               out=None, lse=None, return_lse: bool = True, stage1_only: bool = False,
               stream=None):
    """MLA decode: q_nope [B, H, R], q_pe [B, H, P] (last dim contiguous; may be
    views of one [B, H, R+P] tensor); kv_cache [nb, bs, R+P].  Returns
    (out [B, H, R], lse [B, H])."""
    torch = _torch()
    _dev(kv_cache, block_table, seq_lens, kv_c, k_pe, slot_mapping, workspace, out, lse)
    for t in (q_nope, q_pe):
        _need(t.is_cuda and t.stride(-1) == 1, "q_nope/q_pe must be GPU tensors with a contiguous last dim")
        _need(t.dtype == torch.bfloat16, "MLA decode is bf16 only")
    B, H, R = q_nope.shape
    P = q_pe.shape[2]
    nb, bs, row = kv_cache.shape
    _need(row == R + P, "cache row must be kv_lora_rank + rope_dim")
    if stage1_only:
        out = lse = None
    else:
        if out is None:
            out = torch.empty((B, H, R), dtype=q_nope.dtype, device=q_nope.device)
        if lse is None and return_lse:
            lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    need = mla_decode_workspace_size(B, max_seq_len, bs, H, R, num_splits, stage1_only)
    if workspace is None and need:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q_nope.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_mla_decode(_ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
                                   _ptr(q_pe), q_pe.stride(0), q_pe.stride(1),
                                   _ptr(kv_c), _ptr(k_pe), _ptr(kv_cache), nb, bs,
                                   _ptr(block_table), block_table.shape[1], _ptr(slot_mapping),
                                   _ptr(seq_lens), B, int(max_seq_len), H, R, P, float(scale),
                                   int(num_splits), _ptr(workspace), wbytes, _ptr(out), _ptr(lse),
                                   _stream(stream)))
    if stage1_only:
        n = need // max(1, 4 * B * H * (R + 1))     # the split count the call used
        if workspace is None:
            return torch.empty((B, H, 0, R + 1), dtype=torch.float32, device=q_nope.device)
        return workspace[: B * H * n * (R + 1)].view(B, H, n, R + 1)
    return out, lse


def mla_decode_balanced(q_nope, q_pe, kv_cache, block_table, seq_lens, scale: float,
                        num_ranges: int = 0, workspace=None, out=None, lse=None,
                        return_lse: bool = True, merge: bool = True, stream=None):
    """Token-balanced MLA decode (no latent write).  num_ranges = 0 takes the
    device's CU count.  merge=False runs only the first kernel (see
    ``decode_balanced``).  Returns (out, lse, workspace, num_ranges)."""
    torch = _torch()
    _dev(kv_cache, block_table, seq_lens, workspace, out, lse)
    for t in (q_nope, q_pe):
        _need(t.is_cuda and t.stride(-1) == 1, "q_nope/q_pe must be GPU tensors with a contiguous last dim")
        _need(t.dtype == torch.bfloat16, "MLA decode is bf16 only")
    B, H, R = q_nope.shape
    P = q_pe.shape[2]
    nb, bs, row = kv_cache.shape
    _need(row == R + P, "cache row must be kv_lora_rank + rope_dim")
    nr = int(num_ranges) or device_num_cus()
    if out is None:
        out = torch.empty((B, H, R), dtype=q_nope.dtype, device=q_nope.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    need = decode_balanced_workspace_bytes(B, H, R, nr)
    if workspace is None:
        workspace = torch.empty(max(1, need // 4), dtype=torch.float32, device=q_nope.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(library().pa_mla_decode_balanced(_ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
                                            _ptr(q_pe), q_pe.stride(0), q_pe.stride(1),
                                            _ptr(kv_cache), nb, bs, _ptr(block_table),
                                            block_table.shape[1], _ptr(seq_lens), B, H, R, P,
                                            float(scale), nr, _ptr(workspace), wbytes, _ptr(out),
                                            _ptr(lse), _stream(stream)))
    if merge:
        decode_balanced_merge(workspace, B, H, R, nr, out, lse, stream=stream)
    return out, lse, workspace, nr


def mla_decode_fp8(q_nope, q_pe, kv_cache, block_table, seq_lens, scale: float,
                   kv_scale: float, kv_c=None, k_pe=None, slot_mapping=None, num_ranges: int = 0,
                   workspace=None, out=None, lse=None, return_lse: bool = True, stream=None):
    """MLA decode over an FP8 latent cache [nb, bs, R + 64] uint8 (one scale
    for the row), token-balanced schedule + merge; q_nope [B, H, R], q_pe
    [B, H, 64] bf16.  Returns (out [B, H, R], lse [B, H])."""
    torch = _torch()
    _dev(kv_cache, block_table, seq_lens, kv_c, k_pe, slot_mapping, workspace, out, lse)
    _fp8_cache(kv_cache)
    for t in (q_nope, q_pe):
        _need(t.is_cuda and t.stride(-1) == 1, "q_nope/q_pe must be GPU tensors with a contiguous last dim")
        _need(t.dtype == torch.bfloat16, "q must be bf16")
    B, H, R = q_nope.shape
    P = q_pe.shape[2]
    nb, bs, row = kv_cache.shape
    _need(row == R + P, "cache row must be kv_lora_rank + rope_dim")
    nr = int(num_ranges) or device_num_cus()
    if out is None:
        out = torch.empty((B, H, R), dtype=q_nope.dtype, device=q_nope.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    if workspace is None:
        need = decode_balanced_workspace_bytes(B, H, R, nr)
        workspace = torch.empty(max(1, need // 4), dtype=torch.float32, device=q_nope.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(library().pa_mla_decode_fp8(_ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
                                       _ptr(q_pe), q_pe.stride(0), q_pe.stride(1), _ptr(kv_c),
                                       _ptr(k_pe), _ptr(kv_cache), nb, bs, _ptr(block_table),
                                       block_table.shape[1], _ptr(slot_mapping), _ptr(seq_lens), B,
                                       H, R, P, float(scale), float(kv_scale), nr, _ptr(workspace),
                                       wbytes, _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def mla_prefill_workspace_bytes(num_seqs: int, total_keys: int, num_heads: int) -> int:
    return library().pa_mla_prefill_workspace_bytes(int(num_seqs), int(total_keys), int(num_heads))


def mla_prefill(q, kv_cache, block_table, query_start_loc, seq_lens, w_kv_b, max_query_len: int,
                total_keys: int, scale: float, kv_c=None, k_pe=None, slot_mapping=None,
                workspace=None, out=None, lse=None, return_lse: bool = True, stream=None):
    """MLA prefill in the multi-head form: q [T, H, 192] bf16 (last dim
    contiguous), latent cache [nb, bs, 576], w_kv_b [H * 256, 512] (or
    [H, 256, 512]) bf16; total_keys = sum of seq_lens (host).  Returns
    (out [T, H, 128], lse [T, H])."""
    torch = _torch()
    _dev(kv_cache, block_table, query_start_loc, seq_lens, w_kv_b, kv_c, k_pe, slot_mapping,
         workspace, out, lse)
    _need(q.is_cuda and q.stride(-1) == 1, "q must be a GPU tensor with a contiguous last dim")
    _need(q.dtype == torch.bfloat16 and kv_cache.dtype == torch.bfloat16 and
          w_kv_b.dtype == torch.bfloat16, "bf16 q, cache and weight")
    _int_tensor(block_table, "int32", "block_table")
    _int_tensor(seq_lens, "int32", "seq_lens")
    _int_tensor(query_start_loc, "int32", "query_start_loc")
    T, H, dq = q.shape
    nb, bs, row = kv_cache.shape
    R = w_kv_b.shape[-1]
    _need(w_kv_b.numel() == H * 256 * R, "w_kv_b must be [H * 256, kv_lora_rank]")
    N = seq_lens.numel()
    _need(query_start_loc.numel() == N + 1, "query_start_loc must have num_seqs + 1 entries")
    if out is None:
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = mla_prefill_workspace_bytes(N, total_keys, H)
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(library().pa_mla_prefill(_ptr(q), q.stride(0), q.stride(1), _ptr(kv_c), _ptr(k_pe),
                                    _ptr(kv_cache), nb, bs, _ptr(block_table), block_table.shape[1],
                                    _ptr(slot_mapping), _ptr(query_start_loc), _ptr(seq_lens), N, T,
                                    int(max_query_len), int(total_keys), _ptr(w_kv_b), H, R,
                                    row - R, dq - (row - R), 256 - (dq - (row - R)), float(scale),
                                    _ptr(workspace), wbytes, _ptr(out), _ptr(lse),
                                    _stream(stream)))
    return out, lse


def lse_merge(part, out_dtype=None, out=None, lse=None, return_lse: bool = True, stream=None):
    """Merge split partials part [R, H, S, Dv+1] (lse last) -> (out [R, H, Dv], lse [R, H])."""
    torch = _torch()
    _dev(part, out, lse)
    _need(part.dtype == torch.float32 and part.dim() == 4, "part must be fp32 [R, H, S, Dv+1]")
    R, H, S, Dv1 = part.shape
    if out is None:
        out = torch.empty((R, H, Dv1 - 1), dtype=out_dtype or torch.float32, device=part.device)
    if lse is None and return_lse:
        lse = torch.empty((R, H), dtype=torch.float32, device=part.device)
    _check(library().pa_lse_merge(_ptr(part), R, H, S, Dv1 - 1, _dtype_code(out), _ptr(out),
                                  _ptr(lse), _stream(stream)))
    return out, lse
