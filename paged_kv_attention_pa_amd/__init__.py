"""Paged KV attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (the C ABI of ``include/pa.h``).
torch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  Importing the package never
loads the library; the first call does, and raises ``PaError`` if it has not
been built (``python -m paged_kv_attention_pa_amd.build``).

Functions mirror the C entry points: ``cache_write``, ``decode``,
``prefill_varlen``, ``mla_decode``, ``lse_merge``, ``decode_balanced``,
``plan_mixed`` + ``mixed_attention`` (a mixed prefill/decode batch),
``plan_cascade`` + ``cascade_attention`` (a batch sharing its first pages),
``cache_write_fp8`` + ``decode_fp8`` + ``prefill_varlen_fp8`` + ``mla_decode_fp8`` (an FP8 E4M3 cache with
per-tensor scales), ``mla_prefill`` (MLA prefill in the multi-head form),
``mla_decode_balanced``, ``decode_balanced_merge``, plus the host helpers ``num_kv_splits``,
``decode_num_kv_splits``, ``mla_num_kv_splits``, ``decode_workspace_bytes``,
``decode_balanced_num_ranges``, ``decode_balanced_workspace_bytes``,
``device_num_cus``.
"""

from ._binding import (  # noqa: F401
    PA_BF16, PA_F32, PA_LAYOUT_KV, PA_LAYOUT_MLA, PaError, EXPORTED_SYMBOLS,
    cache_write, decode, decode_balanced, decode_balanced_merge, decode_num_kv_splits,
    decode_balanced_num_ranges, decode_balanced_workspace_bytes,
    decode_workspace_bytes, decode_workspace_size, mla_decode_workspace_size, decode_noalloc,
    NOALLOC_SCRATCH_BYTES, device_num_cus, last_error, MixedPlan, mixed_attention, plan_mixed,
    CascadePlan, cascade_attention, plan_cascade, cache_write_fp8, decode_fp8,
    mla_decode_fp8, mla_prefill, mla_prefill_workspace_bytes, prefill_varlen_fp8,
    library, library_path, lse_merge, mla_decode, mla_decode_balanced, mla_num_kv_splits,
    num_kv_splits, prefill_varlen,
)

__version__ = "0.1.0"
