// Host-side launchers of the gfx950 kernels.  The C entry points in api.cpp
// validate arguments and then call these; each launcher only sizes a grid and
// enqueues on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// ----------------------------------------------------------- cache write
struct CacheWriteKV {
  const void* k; int64_t k_stride;   // elements between tokens
  const void* v; int64_t v_stride;
  void* cache; int64_t num_blocks; int block_size; int num_kv_heads; int head_dim;
  const int64_t* slots; int num_tokens;
  int elem_bytes;                    // 2 (bf16) or 4 (fp32)
};
hipError_t launch_cache_write_kv(const CacheWriteKV& a, hipStream_t s);

struct CacheWriteMLA {
  const void* kv_c; int64_t c_stride;
  const void* k_pe; int64_t p_stride;
  void* cache; int64_t num_blocks; int block_size; int rank; int rope;
  const int64_t* slots; int num_tokens;
};
hipError_t launch_cache_write_mla(const CacheWriteMLA& a, hipStream_t s);

// FP8 (E4M3) cache writes: bf16 rows in, code = E4M3(x / scale) stored.
// GQA layout [nb, 2, bs, Hkv, D] (K with k_scale, V with v_scale); MLA layout
// [nb, bs, rank + rope] with one scale for the row (k_scale).
struct CacheWriteFp8 {
  int mla;
  const void* k; int64_t k_stride;   // GQA k or MLA kv_c; stride in elements
  const void* v; int64_t v_stride;   // GQA v or MLA k_pe
  void* cache; int64_t num_blocks; int block_size;
  int num_kv_heads; int head_dim;    // GQA
  int rank; int rope;                // MLA
  const int64_t* slots; int num_tokens;
  float k_scale; float v_scale;
};
hipError_t launch_cache_write_fp8(const CacheWriteFp8& a, hipStream_t s);

// ---------------------------------------------------------------- decode
struct DecodeGQA {
  int bf16;                      // 1: bf16 storage, 0: fp32
  const void* q;                 // [B, Hq, D]
  const void* cache;             // [nb, 2, bs, Hkv, D]
  int64_t num_blocks; int block_size;
  const int32_t* block_table; int max_blocks;
  const int32_t* seq_lens; int num_seqs;
  int num_q_heads; int num_kv_heads; int head_dim;
  float scale;
  int num_splits; int split_tokens;  // S and P: split s covers [s P, (s+1) P)
  int direct;                    // 1: S == 1, write out/lse directly
  float* part;                   // [B, Hq, S, D+1] when !direct; empty splits get lse -inf
  void* out; float* lse;         // final outputs (direct mode)
};
hipError_t launch_decode_gqa(const DecodeGQA& a, hipStream_t s);

// Merge of split partials [R, H, S, Dv+1]; splits with lse -inf weigh 0.
struct LseMerge {
  const float* part; int num_rows; int num_heads; int num_splits; int head_dim_v;
  int out_bf16; void* out; float* lse;
};
hipError_t launch_lse_merge(const LseMerge& a, hipStream_t s);

// Token-balanced decode (bf16, head_dim 128): range j of num_ranges covers
// chunks [j T / nr, (j+1) T / nr) of the concatenated 32-token chunk list,
// nr = min(num_ranges, T) (balanced.hpp).  Requests inside one range go to
// out/lse; the others leave one segment per range in
// part[(j + r) * Hq + head][Dv + 4] (values 0..Dv-1, lse at Dv).  cu[B + 1]
// receives the chunk prefix sums.
struct DecodeBalanced {
  const void* q; const void* cache;
  int64_t num_blocks; int block_size;
  const int32_t* block_table; int max_blocks;
  const int32_t* seq_lens; int num_seqs; int len_cap;   // len_cap = max_blocks * block_size
  int num_q_heads; int num_kv_heads;
  float scale;
  int num_ranges;
  int32_t* cu; float* part;
  void* out; float* lse;
  // FP8 (E4M3) cache: keys are code * k_scale, values code * v_scale
  int fp8; float k_scale; float v_scale;
  // bf16 only: the step's new tokens, k_new / v_new [num_seqs, Hkv, 128],
  // written by the kernel itself to slots[r] (NULL: no write)
  const void* k_new; const void* v_new; const int64_t* slots;
};
hipError_t launch_decode_balanced(const DecodeBalanced& a, hipStream_t s);

struct BalancedMerge {
  const int32_t* cu; const float* part;
  int num_seqs; int num_q_heads; int head_dim; int num_ranges;   // head_dim 128 or 512
  void* out; float* lse;
};
hipError_t launch_balanced_merge(const BalancedMerge& a, hipStream_t s);

int balanced_num_ranges(int num_kv_heads, int num_cus);   // ranges for 8 waves per CU
// Overhead units per request in the MLA decode's balanced list (a request
// switch costs about five 32-key tiles); the GQA decode's list has none.
constexpr int kMlaRangeOverhead = 5;
size_t balanced_cu_bytes(int num_seqs);                    // cu[] size, 256-B aligned

// ------------------------------------------------------------------- MLA
// MLA decode.  num_ranges = 0: per-request splits (num_splits, split_tokens,
// direct; partials [B, H, S, 513]).  num_ranges > 0: token-balanced ranges
// (balanced.hpp; segment rows [(nr + B) H, 516], prefix sums in cu).
struct MlaDecode {
  const void* q_nope; int64_t qn_sb, qn_sh;
  const void* q_pe; int64_t qp_sb, qp_sh;
  const void* cache; int64_t num_blocks; int block_size;
  const int32_t* block_table; int max_blocks;
  const int32_t* seq_lens; int num_seqs;
  int num_heads; int rank; int rope;
  float scale;
  int num_splits; int split_tokens; int direct;
  float* part; void* out; float* lse;
  int num_ranges; int32_t* cu;
  int fp8; float kv_scale;   // E4M3 cache, one scale for the row (balanced schedule)
};
hipError_t launch_mla_decode(const MlaDecode& a, hipStream_t s);

// ----------------------------------------------------------- MLA prefill
// Multi-head form: kv_lora_rank 512, rope 64, qk_nope 128, v 128.
struct MlaPrefill {
  const void* q; int64_t q_st, q_sh;        // [T, H, 192] bf16 (element strides)
  const void* cache; int64_t num_blocks; int block_size;   // latent [nb, bs, 576] bf16
  const int32_t* block_table; int max_blocks;
  const int32_t* query_start_loc; const int32_t* seq_lens; int num_seqs;
  int num_tokens; int max_query_len; int total_keys;
  const void* w;                            // kv_b_proj weight [H, 256, 512] bf16
  int num_heads; float scale;
  int32_t* key_start;                       // [N + 1] (workspace)
  void* k_exp; void* v_exp;                 // [total_keys, H, 192], [total_keys, H, 128] (workspace)
  void* out; float* lse;                    // [T, H, 128] bf16, [T, H] fp32 or null
  int32_t* items; int32_t* n_items;         // attention work list [item_cap][2] (request, q tile),
  int item_cap;                             // and its length (workspace)
};
hipError_t launch_mla_prefill(const MlaPrefill& a, hipStream_t s);

// --------------------------------------------------------------- prefill
struct PrefillVarlen {
  const void* q;                  // [T, Hq, D]
  const void* cache;
  int64_t num_blocks; int block_size;
  const int32_t* block_table; int max_blocks;
  const int32_t* query_start_loc; const int32_t* seq_lens;
  int num_seqs; int num_tokens; int max_query_len; int max_seq_len;
  int num_q_heads; int num_kv_heads; int head_dim;
  float scale; int causal;
  void* out; float* lse;
  // Shared-prefix mode (prefix_splits > 0): every query row of the batch
  // (num_tokens rows, no causal mask) against keys [0, prefix_len) of
  // block_table row 0, cut into prefix_splits ranges of split_keys keys
  // (a multiple of 64); fp32 partials part_o [splits, T, Hq, D] (normalised
  // by the range's own sum) and part_lse [splits, T, Hq] (natural log)
  // replace out and lse.
  int prefix_len; int prefix_splits; int split_keys;
  float* part_o; float* part_lse;
  // FP8 (E4M3) cache: keys are code * k_scale, values code * v_scale
  int fp8; float k_scale; float v_scale;
};
hipError_t launch_prefill_varlen(const PrefillVarlen& a, hipStream_t s);

// Cascade attention: per-request key counts past the shared prefix, and the
// merge of the prefix's partials with the suffix's result.
struct SuffixLens {
  const int32_t* seq_lens; int32_t* out; int num_seqs;
  int prefix_len; int max_suffix;   // out[r] = clamp(seq_lens[r] - prefix_len, 0, max_suffix)
};
hipError_t launch_suffix_lens(const SuffixLens& a, hipStream_t s);

struct CascadeMerge {
  const float* part_o;     // [splits, rows, 128] fp32, normalised per split
  const float* part_lse;   // [splits, rows] natural log
  int num_splits;
  const float* suffix_lse; // [rows]
  void* out;               // [rows, 128] bf16: the suffix's result in, the merged result out
  float* lse;              // [rows] or null
  int64_t rows;            // num_tokens * num_q_heads
};
hipError_t launch_cascade_merge(const CascadeMerge& a, hipStream_t s);

// Record a message for pa_last_error() (printf format) and return st.
// Defined with the entry points; for entry points in other sources.
int set_error(int st, const char* fmt, ...);

}  // namespace pa
