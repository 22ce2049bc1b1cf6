// Step 1 of the paged-attention contract ("Attention Backends", "What paged
// attention requires of a kernel"): copy each new token's key/value rows into
// the block-pool cache at slot_mapping[t] (slot = block * block_size + offset).
//
// One thread moves one 16-byte chunk (8 bf16 / 4 fp32), so a 128-wide bf16
// head row is 16 consecutive lanes and every store is a full 16-byte vector
// store.  A fallback instantiation copies single elements when a pointer or
// stride is not 16-byte aligned.  The copy is bit-exact; negative or
// out-of-pool slots are skipped.
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

template <int kVec>
struct Chunk;
template <> struct Chunk<16> { using T = u32x4_t; };
template <> struct Chunk<4> { using T = uint32_t; };
template <> struct Chunk<2> { using T = uint16_t; };

// GQA layout [nb, 2, bs, Hkv, D].
template <int kVec>
__global__ __launch_bounds__(256) void cache_write_kv_kernel(CacheWriteKV a) {
  using C = typename Chunk<kVec>::T;
  const int64_t row_bytes = int64_t(a.head_dim) * a.elem_bytes;
  const int chunks = int(row_bytes / kVec);
  const int64_t per_token = int64_t(a.num_kv_heads) * chunks;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= per_token * a.num_tokens) return;
  const int t = int(i / per_token);
  const int rem = int(i - int64_t(t) * per_token);
  const int h = rem / chunks;
  const int c = rem - h * chunks;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot - blk * a.block_size;
  const int64_t head_row = int64_t(a.num_kv_heads) * row_bytes;    // bytes per token slot
  char* kdst = static_cast<char*>(a.cache) +
               ((blk * 2 + 0) * a.block_size + off) * head_row + h * row_bytes + int64_t(c) * kVec;
  char* vdst = kdst + int64_t(a.block_size) * head_row;
  const char* ksrc = static_cast<const char*>(a.k) +
                     (int64_t(t) * a.k_stride + int64_t(h) * a.head_dim) * a.elem_bytes + int64_t(c) * kVec;
  const char* vsrc = static_cast<const char*>(a.v) +
                     (int64_t(t) * a.v_stride + int64_t(h) * a.head_dim) * a.elem_bytes + int64_t(c) * kVec;
  const C kv = *reinterpret_cast<const C*>(ksrc);
  const C vv = *reinterpret_cast<const C*>(vsrc);
  *reinterpret_cast<C*>(kdst) = kv;
  *reinterpret_cast<C*>(vdst) = vv;
}

// MLA layout [nb, bs, rank + rope]: the row is kv_c then k_pe (bf16).
template <int kVec>
__global__ __launch_bounds__(256) void cache_write_mla_kernel(CacheWriteMLA a) {
  using C = typename Chunk<kVec>::T;
  const int c_chunks = a.rank * 2 / kVec;
  const int p_chunks = a.rope * 2 / kVec;
  const int per_token = c_chunks + p_chunks;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(per_token) * a.num_tokens) return;
  const int t = int(i / per_token);
  const int c = int(i - int64_t(t) * per_token);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;
  const int64_t row_bytes = int64_t(a.rank + a.rope) * 2;
  char* dst = static_cast<char*>(a.cache) + slot * row_bytes + int64_t(c) * kVec;
  const char* src;
  if (c < c_chunks)
    src = static_cast<const char*>(a.kv_c) + int64_t(t) * a.c_stride * 2 + int64_t(c) * kVec;
  else
    src = static_cast<const char*>(a.k_pe) + int64_t(t) * a.p_stride * 2 + int64_t(c - c_chunks) * kVec;
  *reinterpret_cast<C*>(dst) = *reinterpret_cast<const C*>(src);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_cache_write_kv(const CacheWriteKV& a, hipStream_t s) {
  if (a.num_tokens <= 0) return hipSuccess;
  const int64_t row_bytes = int64_t(a.head_dim) * a.elem_bytes;
  const bool vec = aligned16(a.k) && aligned16(a.v) && aligned16(a.cache) &&
                   (row_bytes % 16 == 0) && ((a.k_stride * a.elem_bytes) % 16 == 0) &&
                   ((a.v_stride * a.elem_bytes) % 16 == 0);
  const int kvec = vec ? 16 : a.elem_bytes;
  const int64_t threads = int64_t(a.num_tokens) * a.num_kv_heads * (row_bytes / kvec);
  const dim3 grid(unsigned((threads + 255) / 256)), block(256);
  if (kvec == 16) hipLaunchKernelGGL(cache_write_kv_kernel<16>, grid, block, 0, s, a);
  else if (kvec == 4) hipLaunchKernelGGL(cache_write_kv_kernel<4>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(cache_write_kv_kernel<2>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cache_write_mla(const CacheWriteMLA& a, hipStream_t s) {
  if (a.num_tokens <= 0) return hipSuccess;
  const bool vec = aligned16(a.kv_c) && aligned16(a.k_pe) && aligned16(a.cache) &&
                   ((a.rank * 2) % 16 == 0) && ((a.rope * 2) % 16 == 0) &&
                   ((a.c_stride * 2) % 16 == 0) && ((a.p_stride * 2) % 16 == 0);
  const int kvec = vec ? 16 : 2;
  const int64_t threads = int64_t(a.num_tokens) * ((a.rank + a.rope) * 2 / kvec);
  const dim3 grid(unsigned((threads + 255) / 256)), block(256);
  if (kvec == 16) hipLaunchKernelGGL(cache_write_mla_kernel<16>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(cache_write_mla_kernel<2>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
