// Token-balanced work partition shared by the GQA and MLA decode kernels.
//
// The keys of every request are cut into 32-token chunks (request r has
// ceil(len_r / 32) of them, len_r = seq_lens[r] clamped to the block-table
// capacity) and the chunks of the whole batch are concatenated, request by
// request, into one list of T chunks.  With nr = min(num_ranges, T), range
// j = 0..nr-1 is chunks [floor(j T / nr), floor((j+1) T / nr)): equal work
// whatever the mix of lengths, and never empty.  The chunk prefix sums
// cu[0..B] (cu[B] = T) let a reader recover the ranges a request touches:
// chunk c belongs to range ((c + 1) nr - 1) / T, the largest j with
// floor(j T / nr) <= c (because j T / nr <= c  <=>  j T < (c + 1) nr).
//
// A range leaves one partial ("segment") per request it touches, except for
// requests that lie wholly inside it, which it finishes itself.  Walking the
// list, each new segment advances j or r (or both), so segment (j, r) has the
// unique slot j + r in [0, nr + B - 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.hpp"

namespace pa {

constexpr int kChunkTokens = 32;

__device__ __forceinline__ int clamp_len(int s, int cap) { return s < 0 ? 0 : (s > cap ? cap : s); }
__device__ __forceinline__ int chunks_of(int len) { return (len + kChunkTokens - 1) / kChunkTokens; }

// A chunk of the list: request r, its chunk lc, the request's (clamped)
// length and the list index of its first chunk.
struct ChunkPos {
  int r, lc, len, base;
};

// The chunk after p.  The caller guarantees that one exists (some later
// request has keys), so the scan over empty requests stops inside the batch.
__device__ __forceinline__ ChunkPos next_chunk(ChunkPos p, const int32_t* seq_lens, int cap, int B) {
  if ((p.lc + 1) * kChunkTokens < p.len) {
    ++p.lc;
    return p;
  }
  p.base += chunks_of(p.len);
  int r = min(p.r + 1, B - 1);
  int len = clamp_len(uniform_load(seq_lens + r), cap);
  while (len == 0 && r + 1 < B) {
    ++r;
    len = clamp_len(uniform_load(seq_lens + r), cap);
  }
  p.r = r;
  p.lc = 0;
  p.len = len;
  return p;
}

// Range of a chunk (see above).
__device__ __forceinline__ int range_of_chunk(int c, int nr, int total) {
  return int(((int64_t(c) + 1) * nr - 1) / total);
}

// Work-group prologue: chunk prefix sums by a block scan over seq_lens (every
// work-group computes them; store_cu makes this one also write cu[0..B]),
// then this work-group's range [c0, c1) of range j and the position of chunk
// c0.  Returns false (for the whole work-group) when range j is empty.
// Every thread of the work-group must call it; it contains two barriers.
// s_wave_sum needs blockDim.x / 64 ints of LDS, s_start two.
__device__ __forceinline__ bool balanced_range(const int32_t* seq_lens, int B, int cap,
                                               int num_ranges, int j, bool store_cu, int32_t* cu,
                                               int* s_wave_sum, int* s_start, int& c0, int& c1,
                                               ChunkPos& start) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per = (B + nthr - 1) / nthr;
  const int rb = min(B, tid * per);
  const int re = min(B, rb + per);
  int local = 0;
  for (int r = rb; r < re; ++r) local += chunks_of(clamp_len(seq_lens[r], cap));
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave_sum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < nthr / 64; ++w) {
    const int t = s_wave_sum[w];
    before += w < wave ? t : 0;
    total += t;
  }
  const int excl = before + incl - local;
  if (store_cu) {
    int run = excl;
    for (int r = rb; r < re; ++r) {
      cu[r] = run;
      run += chunks_of(clamp_len(seq_lens[r], cap));
    }
    if (tid == 0) cu[B] = total;
  }
  const int nr = min(num_ranges, total);
  if (j >= nr) return false;   // the same for every thread of the work-group
  c0 = int(int64_t(j) * total / nr);
  c1 = int(int64_t(j + 1) * total / nr);
  if (c0 >= excl && c0 < excl + local) {
    int run = excl;
    for (int r = rb; r < re; ++r) {
      const int n = chunks_of(clamp_len(seq_lens[r], cap));
      if (c0 < run + n) {
        s_start[0] = r;
        s_start[1] = run;
        break;
      }
      run += n;
    }
  }
  __syncthreads();
  start.r = __builtin_amdgcn_readfirstlane(s_start[0]);
  start.base = __builtin_amdgcn_readfirstlane(s_start[1]);
  start.len = clamp_len(uniform_load(seq_lens + start.r), cap);
  start.lc = c0 - start.base;
  return true;
}

}  // namespace pa
