// GQA decode over the paged cache with split-KV partials, and the LSE merge.
//
// Method: "第 1 章 注意力后端" §3.1 (decode reads the whole history with one
// query row; split the history into segments, compute each segment's partial
// output with its softmax normaliser, then merge) and §4.1 (online softmax:
// keep a running max and sum, rescale the accumulated output when a new tile
// raises the max).  Workspace format (B, H, S, D+1), lse in the last slot:
// "Triton 與 MLA", 資料流.
//
// gfx950 mapping.  One work-group of 4 waves owns (request r, KV head h,
// split s) and walks the split's pages in 16-token groups, wave w taking
// groups w, w+4, ...  Within a wave, lane = 16*sub + c: the 16 lanes of a row
// hold one token's 128-wide key (lane c owns dims 8c..8c+7, one 16-byte load
// for bf16), so every load instruction reads four whole 256-byte head rows.
// Each lane keeps the q rows of all G query heads of the group for its 8
// dims and reuses every key/value byte it loads G times from registers.
// The dot products are reduced over the row with four DPP adds; each of the
// 4 rows of a wave runs its own online softmax; the 16 per-wave/per-row
// states are merged once per split through LDS.  Work-group ids put the KV
// heads of one (request, split) next to each other so that the 8 groups
// reading one page run together and share its DRAM rows.
// Decode is HBM-bound (about 4*G flop per cache byte), so the VALU path with
// packed-bf16 dot products is used; no MFMA.
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kGroupTokens = 16;

// One lane's slice of a head row: 8 consecutive elements.
template <bool kBF16> struct Row8;
template <> struct Row8<true> {
  u32x4_t w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = load16(p); }
  __device__ __forceinline__ void zero() { w = u32x4_t{0, 0, 0, 0}; }
  __device__ __forceinline__ float at(int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
};
template <> struct Row8<false> {
  u32x4_t w0, w1;
  __device__ __forceinline__ void load(const float* p) { w0 = load16(p); w1 = load16(p + 4); }
  __device__ __forceinline__ void zero() { w0 = u32x4_t{0, 0, 0, 0}; w1 = w0; }
  __device__ __forceinline__ float at(int e) const {
    return __uint_as_float(e < 4 ? w0[e] : w1[e - 4]);
  }
};

template <bool kBF16>
__device__ __forceinline__ float dot8(const Row8<kBF16>& q, const Row8<kBF16>& k);
template <>
__device__ __forceinline__ float dot8<true>(const Row8<true>& q, const Row8<true>& k) {
  float s = dot2_bf16(q.w[0], k.w[0], 0.0f);
  s = dot2_bf16(q.w[1], k.w[1], s);
  s = dot2_bf16(q.w[2], k.w[2], s);
  return dot2_bf16(q.w[3], k.w[3], s);
}
template <>
__device__ __forceinline__ float dot8<false>(const Row8<false>& q, const Row8<false>& k) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf(q.at(e), k.at(e), s);
  return s;
}

template <bool kBF16> struct Elem;
template <> struct Elem<true> { using T = uint16_t; };
template <> struct Elem<false> { using T = float; };

template <bool kBF16, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeGQA a) {
  using T = typename Elem<kBF16>::T;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;   // 8-element chunk of the head dim
  const int sub = lane >> 4; // token slot within a 4-token load

  // work-group -> (kv head, split, request); heads of one page are adjacent
  const int Hkv = a.num_kv_heads;
  const int S = a.num_splits;
  int id = blockIdx.x;
  const int h = id % Hkv; id /= Hkv;
  const int s = id % S;
  const int r = id / S;

  const int bs = a.block_size;
  const int seq = min(a.seq_lens[r], a.max_blocks * bs);
  const int t0 = s * a.split_tokens;
  const int Hq = a.num_q_heads;
  if (t0 >= seq) {   // empty split: weight 0 in the merge
    if (!a.direct && threadIdx.x < G)
      a.part[((int64_t(r) * Hq + int64_t(h) * G + threadIdx.x) * S + s) * (kD + 1) + kD] = -INFINITY;
    if (a.direct) {  // no key at all: out = 0, lse = -inf
      for (int i = threadIdx.x; i < G * kD; i += blockDim.x) {
        const int64_t o = (int64_t(r) * Hq + int64_t(h) * G) * kD + i;
        if constexpr (kBF16) static_cast<uint16_t*>(a.out)[o] = 0;
        else static_cast<float*>(a.out)[o] = 0.0f;
      }
      if (a.lse && threadIdx.x < G) a.lse[int64_t(r) * Hq + int64_t(h) * G + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int t1 = min(seq, t0 + a.split_tokens);
  const int n_groups = (t1 - t0 + kGroupTokens - 1) / kGroupTokens;

  const float scale2 = a.scale * kLog2e;
  const int64_t tok_stride = int64_t(Hkv) * kD;          // elements between slots
  const int64_t kv_stride = int64_t(bs) * tok_stride;    // K half -> V half
  const T* cache = static_cast<const T*>(a.cache);
  const int32_t* table = a.block_table + int64_t(r) * a.max_blocks;

  Row8<kBF16> qr[G];
  {
    const T* qp = static_cast<const T*>(a.q) + (int64_t(r) * a.num_q_heads + int64_t(h) * G) * kD + 8 * c;
#pragma unroll
    for (int j = 0; j < G; ++j) qr[j].load(qp + j * kD);
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNoMax;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
  }

  auto group_ptr = [&](int g) -> const T* {
    const int tok = t0 + g * kGroupTokens;
    int64_t blk = table[tok / bs];
    blk = (blk < 0 || blk >= a.num_blocks) ? 0 : blk;
    const int off = tok - (tok / bs) * bs;
    return cache + (blk * 2 * bs + off) * tok_stride + int64_t(h) * kD + 8 * c;
  };

  Row8<kBF16> kc[4], vc[4], kn[4], vn[4];
  int g = wave;
  if (g < n_groups) {
    const T* p = group_ptr(g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kc[i].load(p + (4 * i + sub) * tok_stride);
      vc[i].load(p + kv_stride + (4 * i + sub) * tok_stride);
    }
  }
  for (; g < n_groups; g += kWaves) {
    const int gn = g + kWaves;
    if (gn < n_groups) {
      const T* p = group_ptr(gn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kn[i].load(p + (4 * i + sub) * tok_stride);
        vn[i].load(p + kv_stride + (4 * i + sub) * tok_stride);
      }
    }
    const int tok0 = t0 + g * kGroupTokens;
    const bool tail = tok0 + kGroupTokens > t1;
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      valid[i] = !tail || (tok0 + 4 * i + sub < t1);
      if (!valid[i]) vc[i].zero();  // stale slots may hold NaN
    }
    float sc[4][G];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float d = row16_sum(dot8<kBF16>(qr[j], kc[i]));
        sc[i][j] = valid[i] ? d * scale2 : -INFINITY;
      }
    float vf[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[i][e] = vc[i].at(e);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mx = fmaxf(fmaxf(sc[0][j], sc[1][j]), fmaxf(sc[2][j], sc[3][j]));
      const float mn = fmaxf(m[j], mx);
      const float alpha = fast_exp2(m[j] - mn);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i][j] - mn);
      m[j] = mn;
      l[j] = fmaf(l[j], alpha, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[j][e] * alpha;
        x = fmaf(p[0], vf[0][e], x);
        x = fmaf(p[1], vf[1][e], x);
        x = fmaf(p[2], vf[2][e], x);
        acc[j][e] = fmaf(p[3], vf[3][e], x);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; }
  }

  // merge the 4 rows of the wave (lanes ^16, ^32 hold the other rows)
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mm = fmaxf(m[j], lane_xor(m[j], 16));
    mm = fmaxf(mm, lane_xor(mm, 32));
    const float f = fast_exp2(m[j] - mm);
    float lj = l[j] * f;
    lj += lane_xor(lj, 16);
    lj += lane_xor(lj, 32);
    l[j] = lj;
    m[j] = mm;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[j][e] * f;
      x += lane_xor(x, 16);
      x += lane_xor(x, 32);
      acc[j][e] = x;
    }
  }

  // merge the 4 waves through LDS
  __shared__ float s_acc[kWaves][G][kD];
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
  if (sub == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][j][8 * c + e] = acc[j][e];
      if (c == 0) { s_m[wave][j] = m[j]; s_l[wave][j] = l[j]; }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += blockDim.x) {
    const int j = idx / kD;
    const int d = idx - j * kD;
    float mm = s_m[0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, s_m[w][j]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][j] - mm);
      num = fmaf(f, s_acc[w][j][d], num);
      den = fmaf(f, s_l[w][j], den);
    }
    const float o = num / den;
    const float lse_nat = (mm + fast_log2(den)) * kLn2;
    const int64_t row = int64_t(r) * Hq + int64_t(h) * G + j;
    if (a.direct) {
      if constexpr (kBF16) static_cast<uint16_t*>(a.out)[row * kD + d] = f32_to_bf16(o);
      else static_cast<float*>(a.out)[row * kD + d] = o;
      if (d == 0 && a.lse) a.lse[row] = lse_nat;
    } else {
      float* pp = a.part + (row * S + s) * (kD + 1);
      pp[d] = o;
      if (d == 0) pp[kD] = lse_nat;
    }
  }
}

// One work-group of 256 threads per (row, head).  Threads first reduce the
// splits' lse to M and keep the weights exp(lse_s - M) in LDS; then lane
// l of wave w accumulates dims l, l + 64, ... over splits w, w + 4, ...
// (each wave-wide load reads 64 consecutive floats of one split row) and the
// four waves' sums are added through LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxDv = 1024;
constexpr int kMergeWChunk = 1024;   // weights held in LDS per pass over the splits

__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(LseMerge a) {
  __shared__ float s_w[kMergeWChunk];
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ float s_acc[3][kMergeMaxDv];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t pair = blockIdx.x;
  const int n = a.num_splits;
  const int Dv = a.head_dim_v;
  const int64_t stride = Dv + 1;
  const float* base = a.part + pair * int64_t(n) * stride;

  // M = max_s lse_s
  float mx = -INFINITY;
  for (int s = tid; s < n; s += kMergeThreads) mx = fmaxf(mx, base[s * stride + Dv]);
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float* out_f = static_cast<float*>(a.out) + pair * Dv;
  uint16_t* out_b = static_cast<uint16_t*>(a.out) + pair * Dv;
  if (mx == -INFINITY) {   // every split empty
    for (int d = tid; d < Dv; d += kMergeThreads) {
      if (a.out_bf16) out_b[d] = 0; else out_f[d] = 0.0f;
    }
    if (tid == 0 && a.lse) a.lse[pair] = -INFINITY;
    return;
  }
  const float mx2 = mx * kLog2e;

  constexpr int kPer = kMergeMaxDv / 64;   // dims per lane, upper bound
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.0f;
  float den = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kMergeWChunk) {
    const int cn = min(kMergeWChunk, n - c0);
    __syncthreads();   // previous chunk's weights no longer read
    for (int s = tid; s < cn; s += kMergeThreads) {
      const float ls = base[(c0 + s) * stride + Dv];
      const float w = (ls == -INFINITY) ? 0.0f : fast_exp2(fmaf(ls, kLog2e, -mx2));
      s_w[s] = w;
      den += w;
    }
    __syncthreads();
    for (int s = wave; s < cn; s += 4) {
      const float w = s_w[s];
      if (w == 0.0f) continue;   // empty split: its output is never read
      const float* row = base + (c0 + s) * stride;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int d = lane + 64 * i;
        if (d < Dv) acc[i] = fmaf(w, row[d], acc[i]);
      }
    }
  }
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  __syncthreads();
  if (lane == 0) s_red[wave] = den;
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int d = lane + 64 * i;
      if (d < Dv) s_acc[wave - 1][d] = acc[i];
    }
  }
  __syncthreads();
  if (wave == 0) {
    den = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    const float inv = 1.0f / den;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int d = lane + 64 * i;
      if (d < Dv) {
        const float o = (acc[i] + s_acc[0][d] + s_acc[1][d] + s_acc[2][d]) * inv;
        if (a.out_bf16) out_b[d] = f32_to_bf16(o); else out_f[d] = o;
      }
    }
    if (lane == 0 && a.lse) a.lse[pair] = mx + fast_log2(den) * kLn2;
  }
}

template <bool kBF16>
hipError_t launch_decode_t(const DecodeGQA& a, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_kv_heads * a.num_splits)), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<kBF16, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<kBF16, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<kBF16, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<kBF16, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gqa(const DecodeGQA& a, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  return a.bf16 ? launch_decode_t<true>(a, s) : launch_decode_t<false>(a, s);
}

hipError_t launch_lse_merge(const LseMerge& a, hipStream_t s) {
  const int64_t pairs = int64_t(a.num_rows) * a.num_heads;
  if (pairs <= 0) return hipSuccess;
  if (a.head_dim_v > kMergeMaxDv || pairs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(unsigned(pairs)), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
