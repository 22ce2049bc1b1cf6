// Cascade (shared-prefix) attention: the two small kernels around the prefix
// and suffix passes ("Attention Backends", section "Cascade attention": the
// blocks every request shares are processed once, the per-request rest
// separately, and the two results combined).
//
// A query row's attention over keys [0, S) is the log-sum-exp combination of
// its attention over the prefix [0, P) and over the suffix [P, S): with
// o_i normalised by their own sums and lse_i = m_i + ln(l_i),
//   o = sum_i exp(lse_i - M) o_i / sum_i exp(lse_i - M),
//   lse = M + ln(sum_i exp(lse_i - M)),   M = max_i lse_i
// ("第 1 章 注意力后端", §3.1 split-KV and §4.1 Figure 5c: partial results
// over disjoint key sets merge exactly).  The prefix arrives as fp32
// partials of several key ranges, the suffix as the bf16 output and fp32 lse
// of the ordinary decode / prefill kernels.
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kRowsPerGroup = 8;   // 32 lanes per row, 4 dims per lane

__global__ __launch_bounds__(256) void suffix_lens_kernel(SuffixLens a) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.num_seqs) return;
  a.out[r] = min(max(a.seq_lens[r] - a.prefix_len, 0), a.max_suffix);
}

__global__ __launch_bounds__(256) void cascade_merge_kernel(CascadeMerge a) {
  const int64_t row = int64_t(blockIdx.x) * kRowsPerGroup + (threadIdx.x >> 5);
  if (row >= a.rows) return;
  const int d = 4 * (threadIdx.x & 31);
  const int n = a.num_splits;
  const float ls = a.suffix_lse[row];
  float mx = ls;
  for (int s = 0; s < n; ++s) mx = fmaxf(mx, a.part_lse[s * a.rows + row]);
  uint16_t* op = static_cast<uint16_t*>(a.out) + row * kD + d;
  if (mx == -INFINITY) {   // no key anywhere
    *reinterpret_cast<uint2*>(op) = uint2{0u, 0u};
    if (a.lse && d == 0) a.lse[row] = -INFINITY;
    return;
  }
  const float mx2 = mx * kLog2e;
  const uint2 so = *reinterpret_cast<const uint2*>(op);
  float w = ls == -INFINITY ? 0.0f : fast_exp2(fmaf(ls, kLog2e, -mx2));
  float den = w;
  float acc0 = w * bf16_lo(so.x), acc1 = w * bf16_hi(so.x);
  float acc2 = w * bf16_lo(so.y), acc3 = w * bf16_hi(so.y);
#pragma unroll 4
  for (int s = 0; s < n; ++s) {
    const float l = a.part_lse[s * a.rows + row];
    const f32x4_t o = *reinterpret_cast<const f32x4_t*>(a.part_o + (s * a.rows + row) * kD + d);
    const float ws = l == -INFINITY ? 0.0f : fast_exp2(fmaf(l, kLog2e, -mx2));
    den += ws;
    acc0 = fmaf(ws, o[0], acc0);
    acc1 = fmaf(ws, o[1], acc1);
    acc2 = fmaf(ws, o[2], acc2);
    acc3 = fmaf(ws, o[3], acc3);
  }
  const float inv = 1.0f / den;
  *reinterpret_cast<uint2*>(op) =
      uint2{pack_bf16x2(acc0 * inv, acc1 * inv), pack_bf16x2(acc2 * inv, acc3 * inv)};
  if (a.lse && d == 0) a.lse[row] = mx + fast_log2(den) * kLn2;
}

}  // namespace

hipError_t launch_suffix_lens(const SuffixLens& a, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(suffix_lens_kernel, dim3((a.num_seqs + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cascade_merge(const CascadeMerge& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t groups = (a.rows + kRowsPerGroup - 1) / kRowsPerGroup;
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cascade_merge_kernel, dim3(unsigned(groups)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
