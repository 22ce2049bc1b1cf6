// Cache write of an FP8 (E4M3) KV cache with per-tensor scales: the new bf16
// rows are divided by their scale (fp32, correctly rounded), rounded to the
// nearest E4M3 value (ties to even, saturating at 448) and stored as one byte
// each at slot_mapping[t] ("Attention Backends", "What paged attention
// requires of a kernel", step 1; "Triton 與 MLA", 資料流: the layer's
// k_scale / v_scale, v_scale = k_scale for the latent cache).
//
// One thread converts 8 consecutive elements of one row: a 16-byte load of
// bf16, an 8-byte store of codes; a 128-wide head row is 16 lanes.  Inputs
// whose pointers or strides are not 16-byte aligned take a one-element path.
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

template <bool kVec>
__device__ __forceinline__ void convert_store(const uint16_t* src, uint8_t* dst, float scale) {
  if constexpr (kVec) {
    const u32x4_t w = load16(src);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]) / scale;
      x[2 * i + 1] = bf16_hi(w[i]) / scale;
    }
    *reinterpret_cast<uint2*>(dst) =
        uint2{f32x4_to_fp8(x[0], x[1], x[2], x[3]), f32x4_to_fp8(x[4], x[5], x[6], x[7])};
  } else {
    const float x = bf16_to_f32(*src) / scale;
    *dst = uint8_t(f32x4_to_fp8(x, 0.0f, 0.0f, 0.0f) & 0xffu);
  }
}

// GQA: thread -> (token, head, group of kE elements)
template <bool kVec>
__global__ __launch_bounds__(256) void cache_write_fp8_kv_kernel(CacheWriteFp8 a) {
  constexpr int kE = kVec ? 8 : 1;
  const int groups = a.head_dim / kE;
  const int64_t per_token = int64_t(a.num_kv_heads) * groups;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= per_token * a.num_tokens) return;
  const int t = int(i / per_token);
  const int rem = int(i - int64_t(t) * per_token);
  const int h = rem / groups;
  const int e = (rem - h * groups) * kE;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot - blk * a.block_size;
  const int64_t tok_bytes = int64_t(a.num_kv_heads) * a.head_dim;   // one byte per element
  uint8_t* kdst = static_cast<uint8_t*>(a.cache) + (blk * 2 * a.block_size + off) * tok_bytes +
                  int64_t(h) * a.head_dim + e;
  uint8_t* vdst = kdst + int64_t(a.block_size) * tok_bytes;
  const uint16_t* ksrc = static_cast<const uint16_t*>(a.k) + int64_t(t) * a.k_stride +
                         int64_t(h) * a.head_dim + e;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v) + int64_t(t) * a.v_stride +
                         int64_t(h) * a.head_dim + e;
  convert_store<kVec>(ksrc, kdst, a.k_scale);
  convert_store<kVec>(vsrc, vdst, a.v_scale);
}

// MLA: thread -> (token, group of kE elements of the rank + rope row)
template <bool kVec>
__global__ __launch_bounds__(256) void cache_write_fp8_mla_kernel(CacheWriteFp8 a) {
  constexpr int kE = kVec ? 8 : 1;
  const int c_groups = a.rank / kE;
  const int per_token = (a.rank + a.rope) / kE;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(per_token) * a.num_tokens) return;
  const int t = int(i / per_token);
  const int g = int(i - int64_t(t) * per_token);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;
  uint8_t* dst = static_cast<uint8_t*>(a.cache) + slot * (a.rank + a.rope) + int64_t(g) * kE;
  const uint16_t* src =
      g < c_groups
          ? static_cast<const uint16_t*>(a.k) + int64_t(t) * a.k_stride + int64_t(g) * kE
          : static_cast<const uint16_t*>(a.v) + int64_t(t) * a.v_stride + int64_t(g - c_groups) * kE;
  convert_store<kVec>(src, dst, a.k_scale);
}

inline bool aligned(const void* p, unsigned n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

}  // namespace

hipError_t launch_cache_write_fp8(const CacheWriteFp8& a, hipStream_t s) {
  if (a.num_tokens <= 0) return hipSuccess;
  if (!a.mla) {
    const bool vec = aligned(a.k, 16) && aligned(a.v, 16) && aligned(a.cache, 8) &&
                     a.head_dim % 8 == 0 && a.k_stride % 8 == 0 && a.v_stride % 8 == 0;
    const int64_t threads = int64_t(a.num_tokens) * a.num_kv_heads * (a.head_dim / (vec ? 8 : 1));
    const dim3 grid(unsigned((threads + 255) / 256)), block(256);
    if (vec) hipLaunchKernelGGL(cache_write_fp8_kv_kernel<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(cache_write_fp8_kv_kernel<false>, grid, block, 0, s, a);
  } else {
    const bool vec = aligned(a.k, 16) && aligned(a.v, 16) && aligned(a.cache, 8) &&
                     a.rank % 8 == 0 && a.rope % 8 == 0 && a.k_stride % 8 == 0 &&
                     a.v_stride % 8 == 0 && (a.rank + a.rope) % 8 == 0;
    const int64_t threads = int64_t(a.num_tokens) * ((a.rank + a.rope) / (vec ? 8 : 1));
    const dim3 grid(unsigned((threads + 255) / 256)), block(256);
    if (vec) hipLaunchKernelGGL(cache_write_fp8_mla_kernel<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(cache_write_fp8_mla_kernel<false>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
