// The C entry points of include/pa.h: argument validation, split planning,
// workspace checks, then launches on the caller's stream.  No allocation, no
// synchronisation.  Every check runs before the first launch, so an error
// leaves the stream untouched.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

pa_status_t ok() {
  g_err[0] = '\0';
  return PA_OK;
}

pa_status_t hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define PA_REQUIRE(cond, st, ...) \
  do {                            \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

bool is_pow2_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

bool scale_ok(float s) { return s >= 0.0f && s <= 3.0e38f; }   // finite, not negative

// The balanced GQA kernel's work-groups cover a power-of-two number of KV
// heads (at most 8) of every token row.
bool balanced_heads_ok(int hkv) { return hkv == 1 || hkv == 2 || hkv == 4 || hkv % 8 == 0; }

// Tokens per split for n splits over max_seq_len keys, rounded up to whole
// pages; at least one page.
int split_tokens_for(int max_seq_len, int n, int block_size) {
  int64_t p = (int64_t(max_seq_len) + n - 1) / n;
  p = (p + block_size - 1) / block_size * block_size;
  if (p < block_size) p = block_size;
  return int(p > INT_MAX ? INT_MAX : p);
}

// Number of splits that actually hold keys when every split has P tokens.
int used_splits(int max_seq_len, int P) {
  if (max_seq_len <= 0) return 1;
  return (max_seq_len + P - 1) / P;
}

std::atomic<int> g_cus_cache{0};

pa_status_t check_common_cache(int64_t num_blocks, int block_size,
                               const int32_t* block_table, int max_blocks_per_seq,
                               const int32_t* seq_lens, int num_seqs, int max_seq_len) {
  PA_REQUIRE(num_seqs >= 0, PA_ERR_INVALID, "num_seqs must be >= 0 (got %d)", num_seqs);
  PA_REQUIRE(num_blocks > 0, PA_ERR_INVALID, "num_blocks must be > 0");
  PA_REQUIRE(block_size > 0 && block_size % 16 == 0, PA_ERR_INVALID,
             "block_size must be a positive multiple of 16 (got %d)", block_size);
  PA_REQUIRE(max_blocks_per_seq > 0, PA_ERR_INVALID, "max_blocks_per_seq must be > 0");
  PA_REQUIRE(max_seq_len >= 0, PA_ERR_INVALID, "max_seq_len must be >= 0");
  PA_REQUIRE(int64_t(max_seq_len) <= int64_t(max_blocks_per_seq) * block_size, PA_ERR_INVALID,
             "max_seq_len %d exceeds max_blocks_per_seq * block_size", max_seq_len);
  PA_REQUIRE(num_blocks <= INT64_MAX / (int64_t(block_size) * 4096), PA_ERR_INVALID,
             "num_blocks too large");
  if (num_seqs > 0) {
    PA_REQUIRE(block_table && seq_lens, PA_ERR_INVALID, "block_table and seq_lens must be non-null");
  }
  return PA_OK;
}

// Token-balanced decode: workspace = cu[num_seqs + 1] (256-B aligned), then
// (num_ranges + num_seqs) * num_heads segment rows of head_dim_v + 4 fp32.
size_t balanced_bytes(int num_seqs, int num_heads, int head_dim_v, int num_ranges) {
  if (num_seqs < 0 || num_heads < 0 || head_dim_v < 0 || num_ranges < 1) return 0;
  const unsigned __int128 b = (unsigned __int128)pa::balanced_cu_bytes(num_seqs) +
                              (unsigned __int128)((int64_t)num_ranges + num_seqs) *
                                  (unsigned)num_heads * ((unsigned)head_dim_v + 4u) * 4u;
  if (b > (unsigned __int128)SIZE_MAX) return 0;
  return size_t(b);
}

pa_status_t check_balanced(int num_seqs, int num_heads, int head_dim_v, int max_blocks_per_seq,
                           int block_size, int num_ranges, const void* workspace,
                           size_t workspace_bytes) {
  PA_REQUIRE(num_ranges >= 1 && num_ranges <= (1 << 24), PA_ERR_INVALID,
             "num_ranges must be in [1, 2^24] (got %d)", num_ranges);
  // unit counts (chunks, plus the MLA list's overhead units per request; the
  // merge's row width tells the two lists apart) are summed in int32 on the device
  const int64_t len_cap = int64_t(max_blocks_per_seq) * block_size;
  const int64_t w = head_dim_v == 128 ? 0 : pa::kMlaRangeOverhead;
  PA_REQUIRE(int64_t(num_seqs) * ((len_cap + 31) / 32 + w) <= INT_MAX, PA_ERR_UNSUPPORTED,
             "num_seqs * (max_blocks_per_seq * block_size / 32 + %d) exceeds 2^31 units",
             int(w));
  const size_t need = balanced_bytes(num_seqs, num_heads, head_dim_v, num_ranges);
  PA_REQUIRE(need > 0 && workspace != nullptr && workspace_bytes >= need, PA_ERR_WORKSPACE,
             "workspace of %zu bytes needed for %d ranges (got %zu)", need, num_ranges,
             workspace_bytes);
  PA_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 15) == 0, PA_ERR_INVALID,
             "workspace must be 16-byte aligned");
  return PA_OK;
}

// The schedule pa_decode / pa_mla_decode run for given sizes, and the
// workspace it needs.  One definition serves the entry points and the
// workspace-size queries, so a caller that sizes its workspace with the
// query gets exactly what the call checks for.
struct DecodeSchedule {
  int n = 1;               // splits (fixed partition)
  int P = 0;               // tokens per split
  bool stage1 = false;     // partials only (out == NULL)
  bool direct = false;     // one split covers every request: no partials
  bool balanced = false;   // token-balanced ranges + segment merge
  int nr = 0;              // balanced ranges
  size_t need = 0;         // workspace bytes
};

pa_status_t device_cus(int* cus) {
  *cus = pa_device_num_cus();
  if (*cus <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
  return PA_OK;
}

pa_status_t gqa_decode_schedule(pa_dtype_t dtype, int num_seqs, int max_seq_len, int block_size,
                                int num_q_heads, int num_kv_heads, int head_dim, int num_splits,
                                bool stage1, DecodeSchedule* s) {
  s->n = num_splits;
  int cus = 0;
  if (s->n == 0) {
    pa_status_t st = device_cus(&cus);
    if (st != PA_OK) return st;
    s->n = pa_decode_num_kv_splits(num_seqs, num_kv_heads, max_seq_len, cus);
  }
  s->P = split_tokens_for(max_seq_len, s->n, block_size);
  s->stage1 = stage1;
  s->direct = !stage1 && used_splits(max_seq_len, s->P) == 1;
  // automatic schedule with more than one split's worth of keys:
  // token-balanced ranges instead of per-request splits
  s->balanced = num_splits == 0 && !stage1 && !s->direct && dtype == PA_BF16 &&
                balanced_heads_ok(num_kv_heads);
  s->nr = s->balanced ? pa_decode_balanced_num_ranges(num_kv_heads, cus) : 0;
  if (s->balanced)
    s->need = balanced_bytes(num_seqs, num_q_heads, head_dim, s->nr);
  else if (!s->direct)
    s->need = pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, s->n);
  else
    s->need = 0;
  return PA_OK;
}

pa_status_t mla_decode_schedule(int num_seqs, int max_seq_len, int block_size, int num_heads,
                                int kv_lora_rank, int num_splits, bool stage1,
                                DecodeSchedule* s) {
  s->n = num_splits;
  int cus = 0;
  if (s->n == 0) {
    pa_status_t st = device_cus(&cus);
    if (st != PA_OK) return st;
    s->n = pa_mla_num_kv_splits(num_seqs, max_seq_len, cus);
  }
  s->P = split_tokens_for(max_seq_len, s->n, block_size);
  s->stage1 = stage1;
  s->direct = !stage1 && used_splits(max_seq_len, s->P) == 1;
  // automatic schedule with more than one split: token-balanced ranges, one
  // work-group per compute unit
  s->balanced = num_splits == 0 && !stage1 && !s->direct;
  s->nr = s->balanced ? cus : 0;
  if (s->balanced)
    s->need = balanced_bytes(num_seqs, num_heads, kv_lora_rank, s->nr);
  else if (!s->direct)
    s->need = pa_decode_workspace_bytes(num_seqs, num_heads, kv_lora_rank, s->n);
  else
    s->need = 0;
  return PA_OK;
}

int32_t* balanced_cu(void* ws) { return static_cast<int32_t*>(ws); }
float* balanced_part(void* ws, int num_seqs) {
  return reinterpret_cast<float*>(static_cast<char*>(ws) + pa::balanced_cu_bytes(num_seqs));
}

}  // namespace

namespace pa {
int set_error(int st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace pa

extern "C" {

int pa_num_kv_splits(int max_seq_len, int num_cus) {
  if (num_cus < 1) num_cus = 1;
  int64_t n = (int64_t(max_seq_len) + 511) / 512;
  if (max_seq_len <= 0) n = 1;
  if (n < 1) n = 1;
  const int64_t cap = 2 * int64_t(num_cus);
  return int(n > cap ? cap : n);
}

int pa_decode_num_kv_splits(int num_seqs, int num_kv_heads, int max_seq_len, int num_cus) {
  if (num_cus < 1) num_cus = 1;
  const int rule = pa_num_kv_splits(max_seq_len, num_cus);
  if (rule <= 1) return rule;
  // a batch with fewer (request, KV head) pairs than twice the compute units
  // gets more, shorter splits, each at least 64 keys long
  const int64_t pairs = int64_t(num_seqs < 1 ? 1 : num_seqs) * (num_kv_heads < 1 ? 1 : num_kv_heads);
  int64_t want = (2 * int64_t(num_cus) + pairs - 1) / pairs;
  const int64_t by_len = (int64_t(max_seq_len) + 63) / 64;
  if (want > by_len) want = by_len;
  if (want > 2 * int64_t(num_cus)) want = 2 * int64_t(num_cus);
  return int(want > rule ? want : rule);
}

size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim_v, int num_splits) {
  if (num_seqs < 0 || num_q_heads < 0 || head_dim_v < 0 || num_splits < 0) return 0;
  const unsigned __int128 b = (unsigned __int128)num_seqs * (unsigned)num_q_heads *
                              (unsigned)num_splits * ((unsigned)head_dim_v + 1u) * 4u;
  if (b > (unsigned __int128)SIZE_MAX) return 0;
  return size_t(b);
}

int pa_mla_num_kv_splits(int num_seqs, int max_seq_len, int num_cus) {
  if (num_cus < 1) num_cus = 1;
  if (num_seqs < 1) num_seqs = 1;
  const int cap = pa_num_kv_splits(max_seq_len, num_cus);
  int64_t want = (2 * int64_t(num_cus) + num_seqs - 1) / num_seqs;
  const int64_t pages = (int64_t(max_seq_len) + 63) / 64;
  if (want > pages) want = pages;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return int(want);
}

int pa_device_num_cus(void) {
  int c = g_cus_cache.load(std::memory_order_relaxed);
  if (c > 0) return c;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  g_cus_cache.store(n, std::memory_order_relaxed);
  return n;
}

const char* pa_last_error(void) { return g_err; }

pa_status_t pa_decode_workspace_size(pa_dtype_t dtype, int num_seqs, int max_seq_len,
                                     int block_size, int num_q_heads, int num_kv_heads,
                                     int head_dim, int num_splits, int partials_only,
                                     size_t* bytes) {
  PA_REQUIRE(bytes != nullptr, PA_ERR_INVALID, "bytes must be non-null");
  *bytes = 0;
  PA_REQUIRE(num_seqs >= 0 && max_seq_len >= 0 && num_splits >= 0, PA_ERR_INVALID,
             "num_seqs, max_seq_len and num_splits must be >= 0");
  PA_REQUIRE(block_size > 0 && block_size % 16 == 0, PA_ERR_INVALID,
             "block_size must be a positive multiple of 16 (got %d)", block_size);
  PA_REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && head_dim > 0, PA_ERR_INVALID,
             "head counts and head_dim must be positive");
  DecodeSchedule sc;
  pa_status_t st = gqa_decode_schedule(dtype, num_seqs, max_seq_len, block_size, num_q_heads,
                                       num_kv_heads, head_dim, num_splits, partials_only != 0,
                                       &sc);
  if (st != PA_OK) return st;
  *bytes = sc.need;
  return ok();
}

pa_status_t pa_mla_decode_workspace_size(int num_seqs, int max_seq_len, int block_size,
                                         int num_heads, int kv_lora_rank, int num_splits,
                                         int partials_only, size_t* bytes) {
  PA_REQUIRE(bytes != nullptr, PA_ERR_INVALID, "bytes must be non-null");
  *bytes = 0;
  PA_REQUIRE(num_seqs >= 0 && max_seq_len >= 0 && num_splits >= 0, PA_ERR_INVALID,
             "num_seqs, max_seq_len and num_splits must be >= 0");
  PA_REQUIRE(block_size > 0 && block_size % 16 == 0, PA_ERR_INVALID,
             "block_size must be a positive multiple of 16 (got %d)", block_size);
  PA_REQUIRE(num_heads > 0 && kv_lora_rank > 0, PA_ERR_INVALID,
             "num_heads and kv_lora_rank must be positive");
  DecodeSchedule sc;
  pa_status_t st = mla_decode_schedule(num_seqs, max_seq_len, block_size, num_heads,
                                       kv_lora_rank, num_splits, partials_only != 0, &sc);
  if (st != PA_OK) return st;
  *bytes = sc.need;
  return ok();
}

// ---------------------------------------------------------------------------
pa_status_t pa_cache_write(pa_layout_t layout, pa_dtype_t dtype,
                           const void* k, int64_t k_token_stride,
                           const void* v, int64_t v_token_stride,
                           void* kv_cache, int64_t num_blocks, int block_size,
                           int num_kv_heads, int head_dim,
                           const int64_t* slot_mapping, int num_tokens,
                           hipStream_t stream) {
  PA_REQUIRE(num_tokens >= 0, PA_ERR_INVALID, "num_tokens must be >= 0");
  PA_REQUIRE(dtype == PA_F32 || dtype == PA_BF16, PA_ERR_INVALID, "unknown dtype %d", int(dtype));
  PA_REQUIRE(num_blocks > 0, PA_ERR_INVALID, "num_blocks must be > 0");
  PA_REQUIRE(block_size > 0 && block_size % 16 == 0, PA_ERR_INVALID,
             "block_size must be a positive multiple of 16 (got %d)", block_size);
  PA_REQUIRE(head_dim > 0 && num_kv_heads > 0, PA_ERR_INVALID, "head_dim and num_kv_heads must be > 0");
  if (num_tokens == 0) return ok();
  PA_REQUIRE(k && v && kv_cache && slot_mapping, PA_ERR_INVALID, "k, v, kv_cache and slot_mapping must be non-null");
  if (layout == PA_LAYOUT_KV) {
    PA_REQUIRE(k_token_stride >= int64_t(num_kv_heads) * head_dim &&
               v_token_stride >= int64_t(num_kv_heads) * head_dim, PA_ERR_INVALID,
               "token strides must be >= num_kv_heads * head_dim");
    pa::CacheWriteKV a{k, k_token_stride, v, v_token_stride, kv_cache, num_blocks, block_size,
                       num_kv_heads, head_dim, slot_mapping, num_tokens, dtype == PA_BF16 ? 2 : 4};
    hipError_t e = pa::launch_cache_write_kv(a, stream);
    if (e != hipSuccess) return hip_fail(e, "cache_write_kv launch");
    return ok();
  }
  if (layout == PA_LAYOUT_MLA) {
    PA_REQUIRE(dtype == PA_BF16, PA_ERR_UNSUPPORTED, "the MLA layout is bf16 only");
    PA_REQUIRE(num_kv_heads == 1, PA_ERR_INVALID, "the MLA layout has one KV head");
    PA_REQUIRE(head_dim > 64, PA_ERR_INVALID, "MLA head_dim must be kv_lora_rank + 64");
    const int rank = head_dim - 64;
    PA_REQUIRE(k_token_stride >= rank && v_token_stride >= 64, PA_ERR_INVALID,
               "token strides must cover kv_lora_rank / rope_dim");
    pa::CacheWriteMLA a{k, k_token_stride, v, v_token_stride, kv_cache, num_blocks, block_size,
                        rank, 64, slot_mapping, num_tokens};
    hipError_t e = pa::launch_cache_write_mla(a, stream);
    if (e != hipSuccess) return hip_fail(e, "cache_write_mla launch");
    return ok();
  }
  return fail(PA_ERR_INVALID, "unknown layout %d", int(layout));
}

// ---------------------------------------------------------------------------
static pa_status_t decode_balanced_impl(const void* q, const void* kv_cache, int64_t num_blocks,
                                        int block_size, const int32_t* block_table,
                                        int max_blocks_per_seq, const int32_t* seq_lens,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, float scale, int num_ranges, void* workspace,
                                        size_t workspace_bytes, void* out, float* lse,
                                        const void* k_new, const void* v_new,
                                        const int64_t* slots, hipStream_t stream);

pa_status_t pa_decode(pa_dtype_t dtype,
                      const void* q, const void* k, const void* v,
                      void* kv_cache, int64_t num_blocks, int block_size,
                      const int32_t* block_table, int max_blocks_per_seq,
                      const int64_t* slot_mapping,
                      const int32_t* seq_lens, int num_seqs, int max_seq_len,
                      int num_q_heads, int num_kv_heads, int head_dim,
                      float scale, int num_splits,
                      void* workspace, size_t workspace_bytes,
                      void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(dtype == PA_F32 || dtype == PA_BF16, PA_ERR_INVALID, "unknown dtype %d", int(dtype));
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, max_seq_len);
  if (st != PA_OK) return st;
  PA_REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0,
             PA_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
             num_q_heads, num_kv_heads);
  PA_REQUIRE(head_dim > 0 && head_dim % 8 == 0 && head_dim <= 256, PA_ERR_INVALID,
             "head_dim must be a multiple of 8 in [8, 256] (got %d)", head_dim);
  PA_REQUIRE(head_dim == 128, PA_ERR_UNSUPPORTED, "decode supports head_dim 128 (got %d)", head_dim);
  PA_REQUIRE(is_pow2_group(num_q_heads / num_kv_heads), PA_ERR_UNSUPPORTED,
             "decode supports num_q_heads / num_kv_heads in {1, 2, 4, 8} (got %d)",
             num_q_heads / num_kv_heads);
  PA_REQUIRE(num_splits >= 0, PA_ERR_INVALID, "num_splits must be >= 0");
  PA_REQUIRE((k == nullptr) == (v == nullptr), PA_ERR_INVALID, "k and v must both be given or both NULL");
  PA_REQUIRE(k == nullptr || slot_mapping != nullptr, PA_ERR_INVALID, "k/v given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || k != nullptr, PA_ERR_INVALID, "slot_mapping given without k/v");
  if (num_seqs == 0) return ok();
  PA_REQUIRE(q && kv_cache, PA_ERR_INVALID, "q and kv_cache must be non-null");
  PA_REQUIRE(out != nullptr || lse == nullptr, PA_ERR_INVALID,
             "lse without out: the partial-only mode (out = NULL) returns no lse");

  DecodeSchedule sc;
  st = gqa_decode_schedule(dtype, num_seqs, max_seq_len, block_size, num_q_heads, num_kv_heads,
                           head_dim, num_splits, out == nullptr, &sc);
  if (st != PA_OK) return st;
  const int n = sc.n, P = sc.P, nr = sc.nr;
  const bool stage1 = sc.stage1, direct = sc.direct, balanced = sc.balanced;
  if (balanced) {
    st = check_balanced(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size, nr,
                        workspace, workspace_bytes);
    if (st != PA_OK) return st;
  } else if (!direct) {
    PA_REQUIRE(workspace != nullptr && workspace_bytes >= sc.need, PA_ERR_WORKSPACE,
               "workspace of %zu bytes needed for %d splits (got %zu)", sc.need, n,
               workspace_bytes);
  }

  // the balanced (bf16) decode writes the new tokens itself; the others
  // after a write kernel
  if (k && !balanced) {
    pa::CacheWriteKV w{k, int64_t(num_kv_heads) * head_dim, v, int64_t(num_kv_heads) * head_dim,
                       kv_cache, num_blocks, block_size, num_kv_heads, head_dim, slot_mapping,
                       num_seqs, dtype == PA_BF16 ? 2 : 4};
    hipError_t e = pa::launch_cache_write_kv(w, stream);
    if (e != hipSuccess) return hip_fail(e, "cache_write_kv launch");
  }
  if (balanced) {
    st = decode_balanced_impl(q, kv_cache, num_blocks, block_size, block_table,
                              max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                              head_dim, scale, nr, workspace, workspace_bytes, out, lse, k, v,
                              slot_mapping, stream);
    if (st != PA_OK) return st;
    return pa_decode_balanced_merge(workspace, workspace_bytes, num_seqs, num_q_heads, head_dim,
                                    nr, out, lse, stream);
  }
  pa::DecodeGQA d{};
  d.bf16 = dtype == PA_BF16;
  d.q = q;
  d.cache = kv_cache;
  d.num_blocks = num_blocks;
  d.block_size = block_size;
  d.block_table = block_table;
  d.max_blocks = max_blocks_per_seq;
  d.seq_lens = seq_lens;
  d.num_seqs = num_seqs;
  d.num_q_heads = num_q_heads;
  d.num_kv_heads = num_kv_heads;
  d.head_dim = head_dim;
  d.scale = scale;
  d.num_splits = direct ? 1 : n;
  d.split_tokens = P;
  d.direct = direct;
  d.part = static_cast<float*>(workspace);
  d.out = out;
  d.lse = lse;
  hipError_t e = pa::launch_decode_gqa(d, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (!direct && !stage1) {
    pa::LseMerge m{static_cast<const float*>(workspace), num_seqs, num_q_heads, n, head_dim,
                   dtype == PA_BF16, out, lse};
    e = pa::launch_lse_merge(m, stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return ok();
}

// ---------------------------------------------------------------------------
int pa_decode_balanced_num_ranges(int num_kv_heads, int num_cus) {
  return pa::balanced_num_ranges(num_kv_heads, num_cus);
}

size_t pa_decode_balanced_workspace_bytes(int num_seqs, int num_heads, int head_dim_v,
                                          int num_ranges) {
  return balanced_bytes(num_seqs, num_heads, head_dim_v, num_ranges);
}

// The balanced decode; with k_new (bf16 [num_seqs, Hkv, 128], v_new alike)
// the kernel also writes the step's new tokens to their slots first.
static pa_status_t decode_balanced_impl(const void* q, const void* kv_cache, int64_t num_blocks,
                                        int block_size, const int32_t* block_table,
                                        int max_blocks_per_seq, const int32_t* seq_lens,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, float scale, int num_ranges, void* workspace,
                                        size_t workspace_bytes, void* out, float* lse,
                                        const void* k_new, const void* v_new,
                                        const int64_t* slots, hipStream_t stream) {
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  PA_REQUIRE(num_seqs >= 0, PA_ERR_INVALID, "num_seqs must be >= 0 (got %d)", num_seqs);
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, 0);
  if (st != PA_OK) return st;
  PA_REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0,
             PA_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
             num_q_heads, num_kv_heads);
  PA_REQUIRE(head_dim == 128, PA_ERR_UNSUPPORTED, "balanced decode supports head_dim 128 (got %d)",
             head_dim);
  PA_REQUIRE(is_pow2_group(num_q_heads / num_kv_heads), PA_ERR_UNSUPPORTED,
             "balanced decode supports num_q_heads / num_kv_heads in {1, 2, 4, 8} (got %d)",
             num_q_heads / num_kv_heads);
  PA_REQUIRE(balanced_heads_ok(num_kv_heads), PA_ERR_UNSUPPORTED,
             "balanced decode supports num_kv_heads 1, 2, 4, 8 or a multiple of 8 (got %d)",
             num_kv_heads);
  st = check_balanced(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size, num_ranges,
                      workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  PA_REQUIRE(q && kv_cache && out, PA_ERR_INVALID, "q, kv_cache and out must be non-null");
  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  pa::DecodeBalanced d{q, kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                       seq_lens, num_seqs, int(cap > INT_MAX ? INT_MAX : cap), num_q_heads,
                       num_kv_heads, scale, num_ranges, balanced_cu(workspace),
                       balanced_part(workspace, num_seqs), out, lse};
  d.k_new = k_new;
  d.v_new = v_new;
  d.slots = slots;
  hipError_t e = pa::launch_decode_balanced(d, stream);
  if (e != hipSuccess) return hip_fail(e, "balanced decode launch");
  return ok();
}

pa_status_t pa_decode_balanced(const void* q, const void* kv_cache, int64_t num_blocks,
                               int block_size, const int32_t* block_table,
                               int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                               int num_q_heads, int num_kv_heads, int head_dim, float scale,
                               int num_ranges, void* workspace, size_t workspace_bytes,
                               void* out, float* lse, hipStream_t stream) {
  return decode_balanced_impl(q, kv_cache, num_blocks, block_size, block_table,
                              max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                              head_dim, scale, num_ranges, workspace, workspace_bytes, out, lse,
                              nullptr, nullptr, nullptr, stream);
}

pa_status_t pa_decode_balanced_merge(void* workspace, size_t workspace_bytes, int num_seqs,
                                     int num_heads, int head_dim_v, int num_ranges, void* out,
                                     float* lse, hipStream_t stream) {
  PA_REQUIRE(num_seqs >= 0, PA_ERR_INVALID, "num_seqs must be >= 0 (got %d)", num_seqs);
  PA_REQUIRE(num_heads > 0, PA_ERR_INVALID, "num_heads must be > 0");
  PA_REQUIRE(head_dim_v == 128 || head_dim_v == 256 || head_dim_v == 512, PA_ERR_UNSUPPORTED,
             "balanced merge supports head_dim_v 128 (GQA), 256 and 512 (MLA) (got %d)", head_dim_v);
  PA_REQUIRE(num_ranges >= 1 && num_ranges <= (1 << 24), PA_ERR_INVALID,
             "num_ranges must be in [1, 2^24] (got %d)", num_ranges);
  const size_t need = balanced_bytes(num_seqs, num_heads, head_dim_v, num_ranges);
  PA_REQUIRE(need > 0 && workspace != nullptr && workspace_bytes >= need, PA_ERR_WORKSPACE,
             "workspace of %zu bytes needed for %d ranges (got %zu)", need, num_ranges,
             workspace_bytes);
  if (num_seqs == 0) return ok();
  PA_REQUIRE(out != nullptr, PA_ERR_INVALID, "out must be non-null");
  pa::BalancedMerge m{balanced_cu(workspace), balanced_part(workspace, num_seqs), num_seqs,
                      num_heads, head_dim_v, num_ranges, out, lse};
  hipError_t e = pa::launch_balanced_merge(m, stream);
  if (e != hipSuccess) return hip_fail(e, "balanced merge launch");
  return ok();
}

// ---------------------------------------------------------------------------
pa_status_t pa_prefill_varlen(pa_dtype_t dtype,
                              const void* q, const void* k, const void* v,
                              void* kv_cache, int64_t num_blocks, int block_size,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int64_t* slot_mapping,
                              const int32_t* query_start_loc,
                              const int32_t* seq_lens, int num_seqs,
                              int num_tokens, int max_query_len, int max_seq_len,
                              int num_q_heads, int num_kv_heads, int head_dim,
                              float scale, int causal,
                              void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(dtype == PA_F32 || dtype == PA_BF16, PA_ERR_INVALID, "unknown dtype %d", int(dtype));
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, max_seq_len);
  if (st != PA_OK) return st;
  PA_REQUIRE(num_tokens >= 0 && max_query_len >= 0, PA_ERR_INVALID, "num_tokens and max_query_len must be >= 0");
  PA_REQUIRE(max_query_len <= num_tokens || num_seqs == 0, PA_ERR_INVALID, "max_query_len exceeds num_tokens");
  PA_REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0,
             PA_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
             num_q_heads, num_kv_heads);
  PA_REQUIRE(head_dim > 0 && head_dim % 8 == 0 && head_dim <= 256, PA_ERR_INVALID,
             "head_dim must be a multiple of 8 in [8, 256] (got %d)", head_dim);
  PA_REQUIRE(causal == 0 || causal == 1, PA_ERR_INVALID, "causal must be 0 or 1");
  PA_REQUIRE(dtype == PA_BF16, PA_ERR_UNSUPPORTED, "prefill supports bf16 only");
  PA_REQUIRE(head_dim == 128, PA_ERR_UNSUPPORTED, "prefill supports head_dim 128 (got %d)", head_dim);
  PA_REQUIRE(is_pow2_group(num_q_heads / num_kv_heads), PA_ERR_UNSUPPORTED,
             "prefill supports num_q_heads / num_kv_heads in {1, 2, 4, 8}");
  PA_REQUIRE((k == nullptr) == (v == nullptr), PA_ERR_INVALID, "k and v must both be given or both NULL");
  PA_REQUIRE(k == nullptr || slot_mapping != nullptr, PA_ERR_INVALID, "k/v given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || k != nullptr, PA_ERR_INVALID, "slot_mapping given without k/v");
  if (num_seqs == 0 || num_tokens == 0) return ok();
  PA_REQUIRE(q && kv_cache && out && query_start_loc, PA_ERR_INVALID,
             "q, kv_cache, out and query_start_loc must be non-null");
  if (k) {
    pa::CacheWriteKV w{k, int64_t(num_kv_heads) * head_dim, v, int64_t(num_kv_heads) * head_dim,
                       kv_cache, num_blocks, block_size, num_kv_heads, head_dim, slot_mapping,
                       num_tokens, 2};
    hipError_t e = pa::launch_cache_write_kv(w, stream);
    if (e != hipSuccess) return hip_fail(e, "cache_write_kv launch");
  }
  pa::PrefillVarlen p{q, kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                      query_start_loc, seq_lens, num_seqs, num_tokens, max_query_len, max_seq_len,
                      num_q_heads, num_kv_heads, head_dim, scale, causal, out, lse};
  hipError_t e = pa::launch_prefill_varlen(p, stream);
  if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "prefill kernel not built");
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

// ---------------------------------------------------------------------------
namespace {

pa_status_t check_mla_q(int64_t qn_stride_b, int64_t qn_stride_h, int64_t qp_stride_b,
                        int64_t qp_stride_h, int num_heads, int kv_lora_rank, int rope_dim,
                        float scale) {
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  PA_REQUIRE(kv_lora_rank > 0 && rope_dim > 0, PA_ERR_INVALID, "kv_lora_rank and rope_dim must be > 0");
  PA_REQUIRE((kv_lora_rank == 512 || kv_lora_rank == 256) && rope_dim == 64, PA_ERR_UNSUPPORTED,
             "MLA decode supports kv_lora_rank 512 or 256 + rope_dim 64 (head size 576 or 320; "
             "got %d + %d)", kv_lora_rank, rope_dim);
  PA_REQUIRE(num_heads > 0, PA_ERR_INVALID, "num_heads must be > 0");
  PA_REQUIRE(num_heads % 16 == 0 && num_heads <= 128, PA_ERR_UNSUPPORTED,
             "MLA decode supports num_heads a multiple of 16 up to 128 (got %d)", num_heads);
  PA_REQUIRE(qn_stride_h >= kv_lora_rank && qp_stride_h >= rope_dim &&
             qn_stride_b >= qn_stride_h * num_heads && qp_stride_b >= qp_stride_h * num_heads,
             PA_ERR_INVALID, "q strides do not describe [num_seqs, num_heads, dim] rows");
  PA_REQUIRE(qn_stride_h % 8 == 0 && qp_stride_h % 8 == 0 && qn_stride_b % 8 == 0 &&
             qp_stride_b % 8 == 0, PA_ERR_INVALID, "q strides must be multiples of 8 elements");
  return PA_OK;
}

}  // namespace

pa_status_t pa_mla_decode_balanced(const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                                   const void* q_pe, int64_t qp_stride_b, int64_t qp_stride_h,
                                   const void* kv_cache, int64_t num_blocks, int block_size,
                                   const int32_t* block_table, int max_blocks_per_seq,
                                   const int32_t* seq_lens, int num_seqs, int num_heads,
                                   int kv_lora_rank, int rope_dim, float scale, int num_ranges,
                                   void* workspace, size_t workspace_bytes, void* out,
                                   float* lse, hipStream_t stream) {
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, 0);
  if (st != PA_OK) return st;
  st = check_mla_q(qn_stride_b, qn_stride_h, qp_stride_b, qp_stride_h, num_heads, kv_lora_rank,
                   rope_dim, scale);
  if (st != PA_OK) return st;
  st = check_balanced(num_seqs, num_heads, kv_lora_rank, max_blocks_per_seq, block_size,
                      num_ranges, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  PA_REQUIRE(q_nope && q_pe && kv_cache && out, PA_ERR_INVALID,
             "q_nope, q_pe, kv_cache and out must be non-null");
  pa::MlaDecode d{q_nope, qn_stride_b, qn_stride_h, q_pe, qp_stride_b, qp_stride_h,
                  kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                  seq_lens, num_seqs, num_heads, kv_lora_rank, rope_dim, scale,
                  1, 0, 0, balanced_part(workspace, num_seqs), out, lse,
                  num_ranges, balanced_cu(workspace)};
  hipError_t e = pa::launch_mla_decode(d, stream);
  if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "MLA kernel not built");
  if (e != hipSuccess) return hip_fail(e, "balanced MLA decode launch");
  return ok();
}

pa_status_t pa_mla_decode(const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                          const void* q_pe, int64_t qp_stride_b, int64_t qp_stride_h,
                          const void* kv_c, const void* k_pe,
                          void* kv_cache, int64_t num_blocks, int block_size,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int64_t* slot_mapping,
                          const int32_t* seq_lens, int num_seqs, int max_seq_len,
                          int num_heads, int kv_lora_rank, int rope_dim,
                          float scale, int num_splits,
                          void* workspace, size_t workspace_bytes,
                          void* out, float* lse, hipStream_t stream) {
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, max_seq_len);
  if (st != PA_OK) return st;
  st = check_mla_q(qn_stride_b, qn_stride_h, qp_stride_b, qp_stride_h, num_heads, kv_lora_rank,
                   rope_dim, scale);
  if (st != PA_OK) return st;
  PA_REQUIRE(num_splits >= 0, PA_ERR_INVALID, "num_splits must be >= 0");
  PA_REQUIRE((kv_c == nullptr) == (k_pe == nullptr), PA_ERR_INVALID,
             "kv_c and k_pe must both be given or both NULL");
  PA_REQUIRE(kv_c == nullptr || slot_mapping != nullptr, PA_ERR_INVALID, "kv_c/k_pe given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || kv_c != nullptr, PA_ERR_INVALID, "slot_mapping given without kv_c/k_pe");
  if (num_seqs == 0) return ok();
  PA_REQUIRE(q_nope && q_pe && kv_cache, PA_ERR_INVALID, "q_nope, q_pe and kv_cache must be non-null");
  PA_REQUIRE(out != nullptr || lse == nullptr, PA_ERR_INVALID,
             "lse without out: the partial-only mode (out = NULL) returns no lse");
  DecodeSchedule sc;
  st = mla_decode_schedule(num_seqs, max_seq_len, block_size, num_heads, kv_lora_rank, num_splits,
                           out == nullptr, &sc);
  if (st != PA_OK) return st;
  const int n = sc.n, P = sc.P, cus = sc.nr;
  const bool stage1 = sc.stage1, direct = sc.direct, balanced = sc.balanced;
  if (balanced) {
    st = check_balanced(num_seqs, num_heads, kv_lora_rank, max_blocks_per_seq, block_size, cus,
                        workspace, workspace_bytes);
    if (st != PA_OK) return st;
  } else if (!direct) {
    PA_REQUIRE(workspace != nullptr && workspace_bytes >= sc.need, PA_ERR_WORKSPACE,
               "workspace of %zu bytes needed for %d splits (got %zu)", sc.need, n,
               workspace_bytes);
  }
  if (kv_c) {
    pa::CacheWriteMLA w{kv_c, kv_lora_rank, k_pe, rope_dim, kv_cache, num_blocks, block_size,
                        kv_lora_rank, rope_dim, slot_mapping, num_seqs};
    hipError_t e = pa::launch_cache_write_mla(w, stream);
    if (e != hipSuccess) return hip_fail(e, "cache_write_mla launch");
  }
  if (balanced) {
    st = pa_mla_decode_balanced(q_nope, qn_stride_b, qn_stride_h, q_pe, qp_stride_b, qp_stride_h,
                                kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                                seq_lens, num_seqs, num_heads, kv_lora_rank, rope_dim, scale, cus,
                                workspace, workspace_bytes, out, lse, stream);
    if (st != PA_OK) return st;
    return pa_decode_balanced_merge(workspace, workspace_bytes, num_seqs, num_heads, kv_lora_rank,
                                    cus, out, lse, stream);
  }
  pa::MlaDecode d{q_nope, qn_stride_b, qn_stride_h, q_pe, qp_stride_b, qp_stride_h,
                  kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                  seq_lens, num_seqs, num_heads, kv_lora_rank, rope_dim, scale,
                  direct ? 1 : n, P, direct, static_cast<float*>(workspace), out, lse, 0, nullptr};
  hipError_t e = pa::launch_mla_decode(d, stream);
  if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "MLA kernel not built");
  if (e != hipSuccess) return hip_fail(e, "MLA decode launch");
  if (!direct && !stage1) {
    pa::LseMerge m{static_cast<const float*>(workspace), num_seqs, num_heads, n, kv_lora_rank,
                   1, out, lse};
    e = pa::launch_lse_merge(m, stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return ok();
}

// ---------------------------------------------------------------------------
pa_status_t pa_lse_merge(const float* part, int num_rows, int num_heads,
                         int num_splits, int head_dim_v, pa_dtype_t out_dtype,
                         void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(num_rows >= 0 && num_heads >= 0, PA_ERR_INVALID, "num_rows and num_heads must be >= 0");
  PA_REQUIRE(num_splits >= 1, PA_ERR_INVALID, "num_splits must be >= 1");
  PA_REQUIRE(head_dim_v >= 1 && head_dim_v <= 1024, PA_ERR_UNSUPPORTED,
             "head_dim_v must be in [1, 1024] (got %d)", head_dim_v);
  PA_REQUIRE(out_dtype == PA_F32 || out_dtype == PA_BF16, PA_ERR_INVALID, "unknown dtype %d", int(out_dtype));
  if (num_rows == 0 || num_heads == 0) return ok();
  PA_REQUIRE(part && out, PA_ERR_INVALID, "part and out must be non-null");
  pa::LseMerge m{part, num_rows, num_heads, num_splits, head_dim_v, out_dtype == PA_BF16,
                 out, lse};
  hipError_t e = pa::launch_lse_merge(m, stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

// ---------------------------------------------------------------------------
pa_status_t pa_plan_mixed(const int32_t* qsl, const int32_t* seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int max_blocks_per_seq, int num_cus, pa_mixed_plan_t* plan) {
  PA_REQUIRE(plan != nullptr, PA_ERR_INVALID, "plan must be non-null");
  std::memset(plan, 0, sizeof(*plan));
  PA_REQUIRE(num_seqs >= 0, PA_ERR_INVALID, "num_seqs must be >= 0 (got %d)", num_seqs);
  PA_REQUIRE(num_seqs == 0 || (qsl && seq_lens), PA_ERR_INVALID,
             "query_start_loc and seq_lens (host copies) must be non-null");
  PA_REQUIRE(block_size > 0 && block_size % 16 == 0, PA_ERR_INVALID,
             "block_size must be a positive multiple of 16 (got %d)", block_size);
  PA_REQUIRE(max_blocks_per_seq > 0, PA_ERR_INVALID, "max_blocks_per_seq must be > 0");
  PA_REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0,
             PA_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
             num_q_heads, num_kv_heads);
  PA_REQUIRE(head_dim == 128, PA_ERR_UNSUPPORTED, "mixed batches support head_dim 128 (got %d)",
             head_dim);
  PA_REQUIRE(is_pow2_group(num_q_heads / num_kv_heads), PA_ERR_UNSUPPORTED,
             "num_q_heads / num_kv_heads must be in {1, 2, 4, 8} (got %d)",
             num_q_heads / num_kv_heads);
  PA_REQUIRE(num_cus >= 0, PA_ERR_INVALID, "num_cus must be >= 0");
  int cus = num_cus;
  if (cus == 0) {
    cus = pa_device_num_cus();
    if (cus <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
  }
  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  PA_REQUIRE(num_seqs == 0 || qsl[0] == 0, PA_ERR_INVALID, "query_start_loc[0] must be 0");
  int nd = 0;
  bool in_decode = true;
  pa_mixed_plan_t p{};   // copied to *plan only when every check has passed
  for (int r = 0; r < num_seqs; ++r) {
    const int64_t L = int64_t(qsl[r + 1]) - qsl[r];
    const int S = seq_lens[r];
    PA_REQUIRE(L >= 0, PA_ERR_INVALID, "query_start_loc must be non-decreasing (request %d)", r);
    PA_REQUIRE(S >= L && S <= cap, PA_ERR_INVALID,
               "request %d: seq_len %d must be in [query rows %lld, max_blocks_per_seq * "
               "block_size]", r, S, (long long)L);
    if (in_decode && L == 1) {
      ++nd;
      p.max_decode_seq_len = S > p.max_decode_seq_len ? S : p.max_decode_seq_len;
      continue;
    }
    in_decode = false;
    p.max_query_len = int(L) > p.max_query_len ? int(L) : p.max_query_len;
    p.max_seq_len = S > p.max_seq_len ? S : p.max_seq_len;
  }
  p.num_seqs = num_seqs;
  p.num_tokens = num_seqs ? qsl[num_seqs] : 0;
  p.num_decode = nd;
  p.prefill_tokens = p.num_tokens - nd;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  // the decode group's schedule: pa_decode's automatic choice (bf16)
  p.decode_splits = 1;
  if (nd > 0) {
    const int n = pa_decode_num_kv_splits(nd, num_kv_heads, p.max_decode_seq_len, cus);
    const int P = split_tokens_for(p.max_decode_seq_len, n, block_size);
    if (used_splits(p.max_decode_seq_len, P) > 1) {
      p.decode_splits = n;
      if (balanced_heads_ok(num_kv_heads)) {
        p.decode_ranges = pa_decode_balanced_num_ranges(num_kv_heads, cus);
        p.workspace_bytes = balanced_bytes(nd, num_q_heads, head_dim, p.decode_ranges);
        PA_REQUIRE(int64_t(nd) * ((cap + 31) / 32) <= INT_MAX, PA_ERR_UNSUPPORTED,
                   "decode group too large for the balanced schedule");
      } else {
        p.workspace_bytes = pa_decode_workspace_bytes(nd, num_q_heads, head_dim, n);
      }
      PA_REQUIRE(p.workspace_bytes > 0, PA_ERR_INVALID, "decode workspace size overflows");
    }
  }
  *plan = p;
  return ok();
}

// Checks of a mixed run, all made before anything is enqueued.
static pa_status_t mixed_check(const pa_mixed_plan_t& p, pa_dtype_t dtype, float scale,
                               const void* q, const void* k, const void* v, const void* kv_cache,
                               int64_t num_blocks, const int32_t* block_table,
                               const int64_t* slot_mapping, const int32_t* query_start_loc,
                               const int32_t* seq_lens, const void* workspace,
                               size_t workspace_bytes, const void* out) {
  PA_REQUIRE(dtype == PA_BF16, PA_ERR_UNSUPPORTED, "mixed batches support PA_BF16");
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  const int64_t cap = int64_t(p.max_blocks_per_seq) * p.block_size;
  PA_REQUIRE(p.num_seqs >= 0 && p.num_decode >= 0 && p.num_decode <= p.num_seqs &&
                 p.num_tokens >= p.num_decode && p.prefill_tokens == p.num_tokens - p.num_decode &&
                 p.head_dim == 128 && p.num_q_heads > 0 && p.num_kv_heads > 0 &&
                 p.num_q_heads % p.num_kv_heads == 0 &&
                 is_pow2_group(p.num_q_heads / p.num_kv_heads) && p.decode_splits >= 1 &&
                 p.decode_ranges >= 0 && (p.decode_ranges == 0 || p.decode_splits > 1) &&
                 p.max_query_len >= 0 && p.max_query_len <= p.num_tokens &&
                 p.max_seq_len >= 0 && p.max_seq_len <= cap && p.max_decode_seq_len >= 0 &&
                 p.max_decode_seq_len <= cap,
             PA_ERR_INVALID, "plan is not one made by pa_plan_mixed");
  pa_status_t st = check_common_cache(num_blocks, p.block_size, block_table, p.max_blocks_per_seq,
                                      seq_lens, p.num_seqs, 0);
  if (st != PA_OK) return st;
  PA_REQUIRE((k == nullptr) == (v == nullptr), PA_ERR_INVALID, "k and v must both be given or both NULL");
  PA_REQUIRE(k == nullptr || slot_mapping != nullptr, PA_ERR_INVALID, "k/v given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || k != nullptr, PA_ERR_INVALID, "slot_mapping given without k/v");
  if (p.num_seqs == 0 || p.num_tokens == 0) return ok();
  PA_REQUIRE(q && kv_cache && out && query_start_loc, PA_ERR_INVALID,
             "q, kv_cache, out and query_start_loc must be non-null");
  if (p.num_decode > 0 && p.decode_ranges > 0) {
    st = check_balanced(p.num_decode, p.num_q_heads, p.head_dim, p.max_blocks_per_seq,
                        p.block_size, p.decode_ranges, workspace, workspace_bytes);
    if (st != PA_OK) return st;
  } else if (p.num_decode > 0 && p.decode_splits > 1) {
    const size_t need =
        pa_decode_workspace_bytes(p.num_decode, p.num_q_heads, p.head_dim, p.decode_splits);
    PA_REQUIRE(workspace != nullptr && workspace_bytes >= need, PA_ERR_WORKSPACE,
               "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  }
  return ok();
}

// The attention of a checked mixed run: the decode group with the plan's
// schedule, then the prefill group (query rows stay absolute: same q, out, lse).
static pa_status_t mixed_enqueue(const pa_mixed_plan_t& p, pa_dtype_t dtype, const void* q,
                                 const void* kv_cache, int64_t num_blocks,
                                 const int32_t* block_table, const int32_t* query_start_loc,
                                 const int32_t* seq_lens, float scale, void* workspace,
                                 size_t workspace_bytes, void* out, float* lse,
                                 hipStream_t stream) {
  pa_status_t st = PA_OK;
  if (p.num_decode > 0 && p.decode_ranges > 0) {
    st = pa_decode_balanced(q, kv_cache, num_blocks, p.block_size, block_table,
                            p.max_blocks_per_seq, seq_lens, p.num_decode, p.num_q_heads,
                            p.num_kv_heads, p.head_dim, scale, p.decode_ranges, workspace,
                            workspace_bytes, out, lse, stream);
    if (st != PA_OK) return st;
    st = pa_decode_balanced_merge(workspace, workspace_bytes, p.num_decode, p.num_q_heads,
                                  p.head_dim, p.decode_ranges, out, lse, stream);
    if (st != PA_OK) return st;
  } else if (p.num_decode > 0) {
    st = pa_decode(dtype, q, nullptr, nullptr, const_cast<void*>(kv_cache), num_blocks,
                   p.block_size, block_table, p.max_blocks_per_seq, nullptr, seq_lens,
                   p.num_decode, p.max_decode_seq_len, p.num_q_heads, p.num_kv_heads, p.head_dim,
                   scale, p.decode_splits, workspace, workspace_bytes, out, lse, stream);
    if (st != PA_OK) return st;
  }
  if (p.num_decode < p.num_seqs) {
    const int nd = p.num_decode;
    st = pa_prefill_varlen(dtype, q, nullptr, nullptr, const_cast<void*>(kv_cache), num_blocks,
                           p.block_size, block_table + int64_t(nd) * p.max_blocks_per_seq,
                           p.max_blocks_per_seq, nullptr, query_start_loc + nd, seq_lens + nd,
                           p.num_seqs - nd, p.num_tokens, p.max_query_len, p.max_seq_len,
                           p.num_q_heads, p.num_kv_heads, p.head_dim, scale, 1, out, lse, stream);
    if (st != PA_OK) return st;
  }
  return ok();
}

pa_status_t pa_mixed_attention(const pa_mixed_plan_t* plan, pa_dtype_t dtype,
                               const void* q, const void* k, const void* v,
                               void* kv_cache, int64_t num_blocks,
                               const int32_t* block_table, const int64_t* slot_mapping,
                               const int32_t* query_start_loc, const int32_t* seq_lens,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(plan != nullptr, PA_ERR_INVALID, "plan must be non-null");
  const pa_mixed_plan_t& p = *plan;
  pa_status_t st = mixed_check(p, dtype, scale, q, k, v, kv_cache, num_blocks, block_table,
                               slot_mapping, query_start_loc, seq_lens, workspace,
                               workspace_bytes, out);
  if (st != PA_OK || p.num_seqs == 0 || p.num_tokens == 0) return st;
  if (k) {
    st = pa_cache_write(PA_LAYOUT_KV, dtype, k, int64_t(p.num_kv_heads) * p.head_dim, v,
                        int64_t(p.num_kv_heads) * p.head_dim, kv_cache, num_blocks, p.block_size,
                        p.num_kv_heads, p.head_dim, slot_mapping, p.num_tokens, stream);
    if (st != PA_OK) return st;
  }
  return mixed_enqueue(p, dtype, q, kv_cache, num_blocks, block_table, query_start_loc, seq_lens,
                       scale, workspace, workspace_bytes, out, lse, stream);
}

// ---------------------------------------------------------------------------
// Cascade workspace: suffix lengths [N] int32, suffix lse [T, Hq], prefix
// partial lse [splits, T, Hq], prefix partial out [splits, T, Hq, 128] (fp32),
// then the suffix pass's own workspace; each piece 256-byte aligned.
struct CascadeLayout {
  size_t lens, suffix_lse, part_lse, part_o, suffix_ws, total;
};

static bool cascade_layout(int num_seqs, int num_tokens, int num_q_heads, int head_dim,
                           int splits, size_t suffix_ws, CascadeLayout* L) {
  auto up = [](unsigned __int128 x) { return (x + 255) / 256 * 256; };
  const unsigned __int128 rows = (unsigned __int128)num_tokens * (unsigned)num_q_heads;
  unsigned __int128 off = 0;
  L->lens = 0;
  off = up(off + (unsigned __int128)num_seqs * 4);
  L->suffix_lse = size_t(off);
  off = up(off + rows * 4);
  L->part_lse = size_t(off);
  off = up(off + rows * (unsigned)splits * 4);
  L->part_o = size_t(off);
  off = up(off + rows * (unsigned)splits * (unsigned)head_dim * 4);
  L->suffix_ws = size_t(off);
  off += suffix_ws;
  if (off > (unsigned __int128)(SIZE_MAX / 2)) return false;
  L->total = size_t(off);
  return true;
}

pa_status_t pa_plan_cascade(const int32_t* qsl, const int32_t* seq_lens, int num_seqs,
                            int num_common_prefix_blocks, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int max_blocks_per_seq, int num_cus,
                            pa_cascade_plan_t* plan) {
  PA_REQUIRE(plan != nullptr, PA_ERR_INVALID, "plan must be non-null");
  std::memset(plan, 0, sizeof(*plan));
  pa_cascade_plan_t c{};
  // the whole batch first: every check of a mixed batch
  pa_status_t st = pa_plan_mixed(qsl, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, num_cus, &c.suffix);
  if (st != PA_OK) return st;
  const int P = num_common_prefix_blocks;
  PA_REQUIRE(P >= 0 && (P == 0 || P < max_blocks_per_seq), PA_ERR_INVALID,
             "num_common_prefix_blocks must be in [0, max_blocks_per_seq) (got %d)", P);
  PA_REQUIRE(int64_t(P) * block_size <= INT_MAX, PA_ERR_INVALID, "shared prefix too long");
  const int Lp = P * block_size;
  int cus = num_cus;
  if (cus == 0) {
    cus = pa_device_num_cus();
    if (cus <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
  }
  int32_t* suffix = nullptr;
  if (Lp > 0 && num_seqs > 0) {
    suffix = new (std::nothrow) int32_t[num_seqs];
    if (!suffix) return fail(PA_ERR_INVALID, "out of host memory");
    for (int r = 0; r < num_seqs; ++r) {
      const int L = qsl[r + 1] - qsl[r];
      if (seq_lens[r] - L < Lp) {
        delete[] suffix;
        return fail(PA_ERR_INVALID,
                    "request %d: its queries start at position %d, inside the %d-key shared "
                    "prefix", r, seq_lens[r] - L, Lp);
      }
      suffix[r] = seq_lens[r] - Lp;
    }
    st = pa_plan_mixed(qsl, suffix, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, cus, &c.suffix);
    delete[] suffix;
    if (st != PA_OK) return st;
  }
  c.prefix_blocks = P;
  c.prefix_len = Lp;
  const int T = c.suffix.num_tokens;
  if (Lp == 0 || T == 0) {
    c.workspace_bytes = c.suffix.workspace_bytes;
    *plan = c;
    return ok();
  }
  // prefix pass: about one work-group per compute unit, at least 256 keys
  // (four 64-key tiles) per range
  const int G = num_q_heads / num_kv_heads;
  const int64_t n_qt = (int64_t(T) * G + 127) / 128;
  const int64_t want = (cus + int64_t(num_kv_heads) * n_qt - 1) / (int64_t(num_kv_heads) * n_qt);
  const int max_splits = (Lp + 255) / 256;
  int splits = int(want < 1 ? 1 : (want > max_splits ? max_splits : want));
  c.split_keys = ((Lp + splits - 1) / splits + 63) / 64 * 64;
  c.prefix_splits = (Lp + c.split_keys - 1) / c.split_keys;
  CascadeLayout L;
  PA_REQUIRE(cascade_layout(num_seqs, T, num_q_heads, head_dim, c.prefix_splits,
                            c.suffix.workspace_bytes, &L),
             PA_ERR_INVALID, "cascade workspace size overflows");
  c.workspace_bytes = L.total;
  *plan = c;
  return ok();
}

pa_status_t pa_cascade_attention(const pa_cascade_plan_t* plan, pa_dtype_t dtype,
                                 const void* q, const void* k, const void* v,
                                 void* kv_cache, int64_t num_blocks,
                                 const int32_t* block_table, const int64_t* slot_mapping,
                                 const int32_t* query_start_loc, const int32_t* seq_lens,
                                 float scale, void* workspace, size_t workspace_bytes,
                                 void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(plan != nullptr, PA_ERR_INVALID, "plan must be non-null");
  const pa_cascade_plan_t& c = *plan;
  const pa_mixed_plan_t& p = c.suffix;
  if (c.prefix_len == 0)
    return pa_mixed_attention(&p, dtype, q, k, v, kv_cache, num_blocks, block_table,
                              slot_mapping, query_start_loc, seq_lens, scale, workspace,
                              workspace_bytes, out, lse, stream);
  PA_REQUIRE(c.prefix_blocks > 0 && c.prefix_blocks < p.max_blocks_per_seq &&
                 c.prefix_len == c.prefix_blocks * p.block_size &&
                 (p.num_tokens == 0 ||
                  (c.prefix_splits >= 1 && c.split_keys > 0 && c.split_keys % 64 == 0 &&
                   int64_t(c.prefix_splits) * c.split_keys >= c.prefix_len)),
             PA_ERR_INVALID, "plan is not one made by pa_plan_cascade");
  CascadeLayout L{};
  if (p.num_tokens > 0) {
    PA_REQUIRE(cascade_layout(p.num_seqs, p.num_tokens, p.num_q_heads, p.head_dim,
                              c.prefix_splits, p.workspace_bytes, &L),
               PA_ERR_INVALID, "plan is not one made by pa_plan_cascade");
    PA_REQUIRE(workspace != nullptr && workspace_bytes >= L.total, PA_ERR_WORKSPACE,
               "workspace of %zu bytes needed (got %zu)", L.total, workspace_bytes);
    PA_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255) == 0, PA_ERR_INVALID,
               "workspace must be 256-byte aligned");
  }
  char* ws = static_cast<char*>(workspace);
  const int32_t* suffix_table = block_table ? block_table + c.prefix_blocks : nullptr;
  pa_status_t st = mixed_check(p, dtype, scale, q, k, v, kv_cache, num_blocks, suffix_table,
                               slot_mapping, query_start_loc, seq_lens,
                               ws ? ws + L.suffix_ws : nullptr,
                               workspace_bytes - L.suffix_ws, out);
  if (st != PA_OK || p.num_seqs == 0 || p.num_tokens == 0) return st;
  if (k) {
    st = pa_cache_write(PA_LAYOUT_KV, dtype, k, int64_t(p.num_kv_heads) * p.head_dim, v,
                        int64_t(p.num_kv_heads) * p.head_dim, kv_cache, num_blocks, p.block_size,
                        p.num_kv_heads, p.head_dim, slot_mapping, p.num_tokens, stream);
    if (st != PA_OK) return st;
  }
  // suffix: keys [P bs, seq_len) of each request, through its table from entry P
  int32_t* lens = reinterpret_cast<int32_t*>(ws + L.lens);
  float* suffix_lse = reinterpret_cast<float*>(ws + L.suffix_lse);
  pa::SuffixLens sl{seq_lens, lens, p.num_seqs, c.prefix_len,
                    (p.max_blocks_per_seq - c.prefix_blocks) * p.block_size};
  hipError_t e = pa::launch_suffix_lens(sl, stream);
  if (e != hipSuccess) return hip_fail(e, "suffix length launch");
  st = mixed_enqueue(p, dtype, q, kv_cache, num_blocks, suffix_table, query_start_loc, lens,
                     scale, ws + L.suffix_ws, workspace_bytes - L.suffix_ws, out, suffix_lse,
                     stream);
  if (st != PA_OK) return st;
  // prefix: every query row against the shared pages (row 0 of the table)
  float* part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  float* part_o = reinterpret_cast<float*>(ws + L.part_o);
  pa::PrefillVarlen pv{q, kv_cache, num_blocks, p.block_size, block_table, p.max_blocks_per_seq,
                       query_start_loc, seq_lens, p.num_seqs, p.num_tokens, p.max_query_len,
                       c.prefix_len, p.num_q_heads, p.num_kv_heads, p.head_dim, scale, 0,
                       nullptr, nullptr, c.prefix_len, c.prefix_splits, c.split_keys, part_o,
                       part_lse};
  e = pa::launch_prefill_varlen(pv, stream);
  if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "prefill kernel not built");
  if (e != hipSuccess) return hip_fail(e, "cascade prefix launch");
  pa::CascadeMerge m{part_o, part_lse, c.prefix_splits, suffix_lse, out, lse,
                     int64_t(p.num_tokens) * p.num_q_heads};
  e = pa::launch_cascade_merge(m, stream);
  if (e != hipSuccess) return hip_fail(e, "cascade merge launch");
  return ok();
}

// ---------------------------------------------------------------------------
static bool fp8_scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

// Checks of an FP8 write (no device work).
static pa_status_t check_write_fp8(pa_layout_t layout, const void* k, int64_t k_token_stride,
                                   const void* v, int64_t v_token_stride, const void* kv_cache,
                                   int64_t num_blocks, int block_size, int num_kv_heads,
                                   int head_dim, const int64_t* slot_mapping, int num_tokens,
                                   float k_scale, float v_scale) {
  PA_REQUIRE(num_tokens >= 0, PA_ERR_INVALID, "num_tokens must be >= 0");
  PA_REQUIRE(num_blocks > 0, PA_ERR_INVALID, "num_blocks must be > 0");
  PA_REQUIRE(block_size > 0 && block_size % 16 == 0, PA_ERR_INVALID,
             "block_size must be a positive multiple of 16 (got %d)", block_size);
  PA_REQUIRE(head_dim > 0 && num_kv_heads > 0, PA_ERR_INVALID, "head_dim and num_kv_heads must be > 0");
  PA_REQUIRE(layout == PA_LAYOUT_KV || layout == PA_LAYOUT_MLA, PA_ERR_INVALID, "unknown layout %d",
             int(layout));
  PA_REQUIRE(fp8_scale_ok(k_scale) && (layout == PA_LAYOUT_MLA || fp8_scale_ok(v_scale)),
             PA_ERR_INVALID, "FP8 scales must be finite and > 0");
  if (layout == PA_LAYOUT_KV) {
    PA_REQUIRE(k_token_stride >= int64_t(num_kv_heads) * head_dim &&
                   v_token_stride >= int64_t(num_kv_heads) * head_dim,
               PA_ERR_INVALID, "token strides must be >= num_kv_heads * head_dim");
  } else {
    PA_REQUIRE(num_kv_heads == 1, PA_ERR_INVALID, "the MLA layout has one KV head");
    PA_REQUIRE(head_dim > 64, PA_ERR_INVALID, "MLA head_dim must be kv_lora_rank + 64");
    PA_REQUIRE(k_token_stride >= head_dim - 64 && v_token_stride >= 64, PA_ERR_INVALID,
               "token strides must cover kv_lora_rank / rope_dim");
  }
  if (num_tokens == 0) return ok();
  PA_REQUIRE(k && v && kv_cache && slot_mapping, PA_ERR_INVALID,
             "k, v, kv_cache and slot_mapping must be non-null");
  return ok();
}

static pa_status_t enqueue_write_fp8(pa_layout_t layout, const void* k, int64_t k_token_stride,
                                     const void* v, int64_t v_token_stride, void* kv_cache,
                                     int64_t num_blocks, int block_size, int num_kv_heads,
                                     int head_dim, const int64_t* slot_mapping, int num_tokens,
                                     float k_scale, float v_scale, hipStream_t stream) {
  if (num_tokens == 0) return ok();
  const bool mla = layout == PA_LAYOUT_MLA;
  pa::CacheWriteFp8 a{mla ? 1 : 0, k, k_token_stride, v, v_token_stride, kv_cache, num_blocks,
                      block_size, num_kv_heads, head_dim, mla ? head_dim - 64 : 0, mla ? 64 : 0,
                      slot_mapping, num_tokens, k_scale, mla ? k_scale : v_scale};
  hipError_t e = pa::launch_cache_write_fp8(a, stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 cache write launch");
  return ok();
}

pa_status_t pa_cache_write_fp8(pa_layout_t layout, const void* k, int64_t k_token_stride,
                               const void* v, int64_t v_token_stride, void* kv_cache,
                               int64_t num_blocks, int block_size, int num_kv_heads, int head_dim,
                               const int64_t* slot_mapping, int num_tokens, float k_scale,
                               float v_scale, hipStream_t stream) {
  pa_status_t st = check_write_fp8(layout, k, k_token_stride, v, v_token_stride, kv_cache,
                                   num_blocks, block_size, num_kv_heads, head_dim, slot_mapping,
                                   num_tokens, k_scale, v_scale);
  if (st != PA_OK) return st;
  return enqueue_write_fp8(layout, k, k_token_stride, v, v_token_stride, kv_cache, num_blocks,
                           block_size, num_kv_heads, head_dim, slot_mapping, num_tokens, k_scale,
                           v_scale, stream);
}

pa_status_t pa_prefill_varlen_fp8(const void* q, const void* k, const void* v, void* kv_cache,
                                  int64_t num_blocks, int block_size, const int32_t* block_table,
                                  int max_blocks_per_seq, const int64_t* slot_mapping,
                                  const int32_t* query_start_loc, const int32_t* seq_lens,
                                  int num_seqs, int num_tokens, int max_query_len,
                                  int max_seq_len, int num_q_heads, int num_kv_heads,
                                  int head_dim, float scale, float k_scale, float v_scale,
                                  int causal, void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  PA_REQUIRE(fp8_scale_ok(k_scale) && fp8_scale_ok(v_scale), PA_ERR_INVALID,
             "FP8 scales must be finite and > 0");
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, max_seq_len);
  if (st != PA_OK) return st;
  PA_REQUIRE(num_tokens >= 0 && max_query_len >= 0, PA_ERR_INVALID,
             "num_tokens and max_query_len must be >= 0");
  PA_REQUIRE(max_query_len <= num_tokens || num_seqs == 0, PA_ERR_INVALID,
             "max_query_len exceeds num_tokens");
  PA_REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0,
             PA_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
             num_q_heads, num_kv_heads);
  PA_REQUIRE(causal == 0 || causal == 1, PA_ERR_INVALID, "causal must be 0 or 1");
  PA_REQUIRE(head_dim == 128, PA_ERR_UNSUPPORTED, "FP8 prefill supports head_dim 128 (got %d)",
             head_dim);
  PA_REQUIRE(is_pow2_group(num_q_heads / num_kv_heads), PA_ERR_UNSUPPORTED,
             "FP8 prefill supports num_q_heads / num_kv_heads in {1, 2, 4, 8}");
  PA_REQUIRE((k == nullptr) == (v == nullptr), PA_ERR_INVALID, "k and v must both be given or both NULL");
  PA_REQUIRE(k == nullptr || slot_mapping != nullptr, PA_ERR_INVALID, "k/v given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || k != nullptr, PA_ERR_INVALID, "slot_mapping given without k/v");
  if (num_seqs == 0 || num_tokens == 0) return ok();
  PA_REQUIRE(q && kv_cache && out && query_start_loc, PA_ERR_INVALID,
             "q, kv_cache, out and query_start_loc must be non-null");
  if (k) {
    st = check_write_fp8(PA_LAYOUT_KV, k, int64_t(num_kv_heads) * head_dim, v,
                         int64_t(num_kv_heads) * head_dim, kv_cache, num_blocks, block_size,
                         num_kv_heads, head_dim, slot_mapping, num_tokens, k_scale, v_scale);
    if (st != PA_OK) return st;
    st = enqueue_write_fp8(PA_LAYOUT_KV, k, int64_t(num_kv_heads) * head_dim, v,
                           int64_t(num_kv_heads) * head_dim, kv_cache, num_blocks, block_size,
                           num_kv_heads, head_dim, slot_mapping, num_tokens, k_scale, v_scale,
                           stream);
    if (st != PA_OK) return st;
  }
  pa::PrefillVarlen p{q, kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                      query_start_loc, seq_lens, num_seqs, num_tokens, max_query_len, max_seq_len,
                      num_q_heads, num_kv_heads, head_dim, scale, causal, out, lse};
  p.fp8 = 1;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  hipError_t e = pa::launch_prefill_varlen(p, stream);
  if (e != hipSuccess) return hip_fail(e, "FP8 prefill launch");
  return ok();
}

pa_status_t pa_decode_fp8(const void* q, const void* k, const void* v, void* kv_cache,
                          int64_t num_blocks, int block_size, const int32_t* block_table,
                          int max_blocks_per_seq, const int64_t* slot_mapping,
                          const int32_t* seq_lens, int num_seqs, int num_q_heads,
                          int num_kv_heads, int head_dim, float scale, float k_scale,
                          float v_scale, int num_ranges, void* workspace, size_t workspace_bytes,
                          void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  PA_REQUIRE(fp8_scale_ok(k_scale) && fp8_scale_ok(v_scale), PA_ERR_INVALID,
             "FP8 scales must be finite and > 0");
  PA_REQUIRE(num_seqs >= 0, PA_ERR_INVALID, "num_seqs must be >= 0 (got %d)", num_seqs);
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, 0);
  if (st != PA_OK) return st;
  PA_REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0,
             PA_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
             num_q_heads, num_kv_heads);
  PA_REQUIRE(head_dim == 128, PA_ERR_UNSUPPORTED, "FP8 decode supports head_dim 128 (got %d)",
             head_dim);
  PA_REQUIRE(is_pow2_group(num_q_heads / num_kv_heads), PA_ERR_UNSUPPORTED,
             "FP8 decode supports num_q_heads / num_kv_heads in {1, 2, 4, 8} (got %d)",
             num_q_heads / num_kv_heads);
  PA_REQUIRE(balanced_heads_ok(num_kv_heads), PA_ERR_UNSUPPORTED,
             "FP8 decode supports num_kv_heads 1, 2, 4 or a multiple of 8 (got %d)", num_kv_heads);
  PA_REQUIRE(num_ranges >= 0, PA_ERR_INVALID, "num_ranges must be >= 0");
  PA_REQUIRE((k == nullptr) == (v == nullptr), PA_ERR_INVALID, "k and v must both be given or both NULL");
  PA_REQUIRE(k == nullptr || slot_mapping != nullptr, PA_ERR_INVALID, "k/v given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || k != nullptr, PA_ERR_INVALID, "slot_mapping given without k/v");
  int nr = num_ranges;
  if (nr == 0) {
    const int cus = pa_device_num_cus();
    if (cus <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
    nr = pa_decode_balanced_num_ranges(num_kv_heads, cus);
  }
  st = check_balanced(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size, nr,
                      workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  PA_REQUIRE(q && kv_cache && out, PA_ERR_INVALID, "q, kv_cache and out must be non-null");
  if (k) {
    st = check_write_fp8(PA_LAYOUT_KV, k, int64_t(num_kv_heads) * head_dim, v,
                         int64_t(num_kv_heads) * head_dim, kv_cache, num_blocks, block_size,
                         num_kv_heads, head_dim, slot_mapping, num_seqs, k_scale, v_scale);
    if (st != PA_OK) return st;
    st = enqueue_write_fp8(PA_LAYOUT_KV, k, int64_t(num_kv_heads) * head_dim, v,
                           int64_t(num_kv_heads) * head_dim, kv_cache, num_blocks, block_size,
                           num_kv_heads, head_dim, slot_mapping, num_seqs, k_scale, v_scale,
                           stream);
    if (st != PA_OK) return st;
  }
  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  pa::DecodeBalanced d{q, kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                       seq_lens, num_seqs, int(cap > INT_MAX ? INT_MAX : cap), num_q_heads,
                       num_kv_heads, scale, nr, balanced_cu(workspace),
                       balanced_part(workspace, num_seqs), out, lse, 1, k_scale, v_scale};
  hipError_t e = pa::launch_decode_balanced(d, stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 decode launch");
  return pa_decode_balanced_merge(workspace, workspace_bytes, num_seqs, num_q_heads, head_dim, nr,
                                  out, lse, stream);
}

pa_status_t pa_mla_decode_fp8(const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                              const void* q_pe, int64_t qp_stride_b, int64_t qp_stride_h,
                              const void* kv_c, const void* k_pe, void* kv_cache,
                              int64_t num_blocks, int block_size, const int32_t* block_table,
                              int max_blocks_per_seq, const int64_t* slot_mapping,
                              const int32_t* seq_lens, int num_seqs, int num_heads,
                              int kv_lora_rank, int rope_dim, float scale, float kv_scale,
                              int num_ranges, void* workspace, size_t workspace_bytes, void* out,
                              float* lse, hipStream_t stream) {
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, 0);
  if (st != PA_OK) return st;
  st = check_mla_q(qn_stride_b, qn_stride_h, qp_stride_b, qp_stride_h, num_heads, kv_lora_rank,
                   rope_dim, scale);
  if (st != PA_OK) return st;
  PA_REQUIRE(kv_lora_rank == 512, PA_ERR_UNSUPPORTED,
             "FP8 MLA decode supports kv_lora_rank 512 (got %d)", kv_lora_rank);
  PA_REQUIRE(fp8_scale_ok(kv_scale), PA_ERR_INVALID, "the FP8 scale must be finite and > 0");
  PA_REQUIRE(num_ranges >= 0, PA_ERR_INVALID, "num_ranges must be >= 0");
  PA_REQUIRE((kv_c == nullptr) == (k_pe == nullptr), PA_ERR_INVALID,
             "kv_c and k_pe must both be given or both NULL");
  PA_REQUIRE(kv_c == nullptr || slot_mapping != nullptr, PA_ERR_INVALID,
             "kv_c/k_pe given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || kv_c != nullptr, PA_ERR_INVALID,
             "slot_mapping given without kv_c/k_pe");
  int nr = num_ranges;
  if (nr == 0) {
    nr = pa_device_num_cus();
    if (nr <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
  }
  st = check_balanced(num_seqs, num_heads, kv_lora_rank, max_blocks_per_seq, block_size, nr,
                      workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  PA_REQUIRE(q_nope && q_pe && kv_cache && out, PA_ERR_INVALID,
             "q_nope, q_pe, kv_cache and out must be non-null");
  const int row = kv_lora_rank + rope_dim;
  if (kv_c) {
    st = check_write_fp8(PA_LAYOUT_MLA, kv_c, kv_lora_rank, k_pe, rope_dim, kv_cache, num_blocks,
                         block_size, 1, row, slot_mapping, num_seqs, kv_scale, kv_scale);
    if (st != PA_OK) return st;
    st = enqueue_write_fp8(PA_LAYOUT_MLA, kv_c, kv_lora_rank, k_pe, rope_dim, kv_cache,
                           num_blocks, block_size, 1, row, slot_mapping, num_seqs, kv_scale,
                           kv_scale, stream);
    if (st != PA_OK) return st;
  }
  pa::MlaDecode d{q_nope, qn_stride_b, qn_stride_h, q_pe, qp_stride_b, qp_stride_h,
                  kv_cache, num_blocks, block_size, block_table, max_blocks_per_seq,
                  seq_lens, num_seqs, num_heads, kv_lora_rank, rope_dim, scale,
                  1, 0, 0, balanced_part(workspace, num_seqs), out, lse,
                  nr, balanced_cu(workspace), 1, kv_scale};
  hipError_t e = pa::launch_mla_decode(d, stream);
  if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "MLA kernel not built");
  if (e != hipSuccess) return hip_fail(e, "FP8 MLA decode launch");
  return pa_decode_balanced_merge(workspace, workspace_bytes, num_seqs, num_heads, kv_lora_rank,
                                  nr, out, lse, stream);
}

// ---------------------------------------------------------------------------
// MLA prefill workspace: key offsets [N + 1] int32, projected keys
// [total, H, 192] and values [total, H, 128] bf16, each 256-byte aligned.
// Workspace of pa_mla_prefill: key offsets [N + 1] and the work list's length,
// the work list (one (request, q tile) pair per 128-query tile: at most
// N + T / 128 of them, and T <= total_keys), then the expanded keys and values.
struct MlaPrefillLayout {
  size_t items_off, k_off, v_off, total;
  int item_cap;
};
static bool mla_prefill_layout(int num_seqs, int total_keys, int num_heads, MlaPrefillLayout* l) {
  if (num_seqs < 0 || total_keys < 0 || num_heads <= 0) return false;
  auto up = [](unsigned __int128 x) { return (x + 255) / 256 * 256; };
  const int64_t cap = int64_t(num_seqs) + total_keys / 128 + 1;
  if (cap > INT32_MAX) return false;
  l->item_cap = int(cap);
  unsigned __int128 off = up((unsigned __int128)(num_seqs + 2) * 4);
  l->items_off = size_t(off);
  off = up(off + (unsigned __int128)cap * 8);
  l->k_off = size_t(off);
  off = up(off + (unsigned __int128)total_keys * (unsigned)num_heads * 192 * 2);
  l->v_off = size_t(off);
  off = up(off + (unsigned __int128)total_keys * (unsigned)num_heads * 128 * 2);
  if (off > (unsigned __int128)(SIZE_MAX / 2)) return false;
  l->total = size_t(off);
  return true;
}

size_t pa_mla_prefill_workspace_bytes(int num_seqs, int total_keys, int num_heads) {
  MlaPrefillLayout l;
  return mla_prefill_layout(num_seqs, total_keys, num_heads, &l) ? l.total : 0;
}

pa_status_t pa_mla_prefill(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                           const void* kv_c, const void* k_pe, void* kv_cache,
                           int64_t num_blocks, int block_size, const int32_t* block_table,
                           int max_blocks_per_seq, const int64_t* slot_mapping,
                           const int32_t* query_start_loc, const int32_t* seq_lens, int num_seqs,
                           int num_tokens, int max_query_len, int total_keys,
                           const void* w_kv_b, int num_heads, int kv_lora_rank, int rope_dim,
                           int qk_nope_dim, int v_head_dim, float scale, void* workspace,
                           size_t workspace_bytes, void* out, float* lse, hipStream_t stream) {
  PA_REQUIRE(scale_ok(scale), PA_ERR_INVALID, "scale must be finite and >= 0");
  pa_status_t st = check_common_cache(num_blocks, block_size, block_table, max_blocks_per_seq,
                                      seq_lens, num_seqs, 0);
  if (st != PA_OK) return st;
  PA_REQUIRE(kv_lora_rank > 0 && rope_dim > 0 && qk_nope_dim > 0 && v_head_dim > 0,
             PA_ERR_INVALID, "MLA dims must be > 0");
  PA_REQUIRE(kv_lora_rank == 512 && rope_dim == 64 && qk_nope_dim == 128 && v_head_dim == 128,
             PA_ERR_UNSUPPORTED,
             "MLA prefill supports kv_lora_rank 512, rope 64, qk_nope 128, v 128 (got %d, %d, %d, %d)",
             kv_lora_rank, rope_dim, qk_nope_dim, v_head_dim);
  PA_REQUIRE(num_heads > 0, PA_ERR_INVALID, "num_heads must be > 0");
  PA_REQUIRE(num_tokens >= 0 && max_query_len >= 0 && total_keys >= 0, PA_ERR_INVALID,
             "num_tokens, max_query_len and total_keys must be >= 0");
  PA_REQUIRE(max_query_len <= num_tokens || num_seqs == 0, PA_ERR_INVALID,
             "max_query_len exceeds num_tokens");
  PA_REQUIRE(q_stride_h >= 192 && q_stride_t >= int64_t(num_heads) * q_stride_h, PA_ERR_INVALID,
             "q strides must cover [num_heads, 192] per token");
  PA_REQUIRE(q_stride_t % 8 == 0 && q_stride_h % 8 == 0, PA_ERR_INVALID,
             "q strides must be multiples of 8 elements (16-byte rows)");
  PA_REQUIRE((kv_c == nullptr) == (k_pe == nullptr), PA_ERR_INVALID,
             "kv_c and k_pe must both be given or both NULL");
  PA_REQUIRE(kv_c == nullptr || slot_mapping != nullptr, PA_ERR_INVALID,
             "kv_c/k_pe given without slot_mapping");
  PA_REQUIRE(slot_mapping == nullptr || kv_c != nullptr, PA_ERR_INVALID,
             "slot_mapping given without kv_c/k_pe");
  MlaPrefillLayout lay;
  PA_REQUIRE(mla_prefill_layout(num_seqs, total_keys, num_heads, &lay),
             PA_ERR_INVALID, "workspace size overflows");
  if (num_seqs == 0 || num_tokens == 0) return ok();
  PA_REQUIRE(q && kv_cache && out && query_start_loc && w_kv_b, PA_ERR_INVALID,
             "q, kv_cache, out, query_start_loc and w_kv_b must be non-null");
  PA_REQUIRE(workspace != nullptr && workspace_bytes >= lay.total, PA_ERR_WORKSPACE,
             "workspace of %zu bytes needed (got %zu)", lay.total, workspace_bytes);
  PA_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255) == 0, PA_ERR_INVALID,
             "workspace must be 256-byte aligned");
  PA_REQUIRE(int64_t(total_keys) * num_heads * 192 <= INT64_MAX / 4, PA_ERR_INVALID,
             "total_keys too large");
  if (kv_c) {
    pa::CacheWriteMLA w{kv_c, kv_lora_rank, k_pe, rope_dim, kv_cache, num_blocks, block_size,
                        kv_lora_rank, rope_dim, slot_mapping, num_tokens};
    hipError_t e = pa::launch_cache_write_mla(w, stream);
    if (e != hipSuccess) return hip_fail(e, "MLA latent write launch");
  }
  char* ws = static_cast<char*>(workspace);
  pa::MlaPrefill m{q, q_stride_t, q_stride_h, kv_cache, num_blocks, block_size, block_table,
                   max_blocks_per_seq, query_start_loc, seq_lens, num_seqs, num_tokens,
                   max_query_len, total_keys, w_kv_b, num_heads, scale,
                   reinterpret_cast<int32_t*>(ws), ws + lay.k_off, ws + lay.v_off, out, lse,
                   reinterpret_cast<int32_t*>(ws + lay.items_off),
                   reinterpret_cast<int32_t*>(ws) + num_seqs + 1, lay.item_cap};
  hipError_t e = pa::launch_mla_prefill(m, stream);
  if (e != hipSuccess) return hip_fail(e, "MLA prefill launch");
  return ok();
}

}  // extern "C"
