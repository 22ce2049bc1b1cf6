// Token-balanced work partition shared by the GQA and MLA decode kernels.
//
// The keys of every request are cut into 32-token chunks (request r has
// n_r = ceil(len_r / 32) of them, len_r = seq_lens[r] clamped to the
// block-table capacity).  A request with keys is laid out in one list as W
// overhead units followed by its n_r chunks, request after request (a request
// without keys takes no units); T is the list's length.  With
// nr = min(num_ranges, T), range j = 0..nr-1 is units
// [floor(j T / nr), floor((j+1) T / nr)) and covers the chunks whose units lie
// in it.  W stands for the work a kernel does when a new request starts
// inside its range (emit the previous request's partial, load the next
// query), so ranges with more request starts get fewer chunks: W = 0 for the
// GQA decode, kMlaRangeOverhead for the MLA decode, whose request switch
// costs about as much as five 32-key tiles.  With W > 0 a range that holds
// only overhead units has no chunks and does nothing.  The unit prefix sums
// cu[0..B] (cu[B] = T) let a reader recover the ranges a request touches:
// unit u belongs to range ((u + 1) nr - 1) / T, the largest j with
// floor(j T / nr) <= u (because j T / nr <= u  <=>  j T < (u + 1) nr); the
// chunks of request r are units [cu[r] + W, cu[r + 1]).
//
// A range leaves one partial ("segment") per request it touches, except for
// requests that lie wholly inside it, which it finishes itself.  Walking the
// list, each new segment advances j or r (or both), so segment (j, r) has the
// unique slot j + r in [0, nr + B - 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {

constexpr int kChunkTokens = 32;
// kMlaRangeOverhead (launch.hpp): W of the MLA decode's ranges (see above)

__device__ __forceinline__ int clamp_len(int s, int cap) { return s < 0 ? 0 : (s > cap ? cap : s); }
__device__ __forceinline__ int chunks_of(int len) { return (len + kChunkTokens - 1) / kChunkTokens; }

// A chunk of the list: request r, its chunk lc, the request's (clamped)
// length and the list index (unit) of its first chunk.
struct ChunkPos {
  int r, lc, len, base;
};

// The chunk after p in a list with kW overhead units per request.  The
// caller guarantees that one exists (some later request has keys), so the
// scan over empty requests stops inside the batch.
template <int kW = 0>
__device__ __forceinline__ ChunkPos next_chunk(ChunkPos p, const int32_t* seq_lens, int cap, int B) {
  if ((p.lc + 1) * kChunkTokens < p.len) {
    ++p.lc;
    return p;
  }
  p.base += chunks_of(p.len) + kW;
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

// Range of a unit of the list (see above).
__device__ __forceinline__ int range_of_unit(int u, int nr, int total) {
  return int(((int64_t(u) + 1) * nr - 1) / total);
}

// Units of request r's list entry: kW + n_r, or none without keys.
template <int kW>
__device__ __forceinline__ int units_of(int len) {
  const int n = chunks_of(len);
  return n > 0 ? n + kW : 0;
}

// Work-group prologue: unit prefix sums by a block scan over seq_lens (every
// work-group computes them; store_cu makes this one also write cu[0..B]),
// then range j's units [c0, c1), the number of chunks in it and the position
// of its first chunk.  Returns false (for the whole work-group) when range j
// is empty or holds no chunk.  Every thread of the work-group must call it;
// it contains two barriers.  s_wave_sum needs blockDim.x / 64 ints of LDS
// (twice that with kW > 0), s_start two.
template <int kW = 0>
__device__ __forceinline__ bool balanced_range(const int32_t* seq_lens, int B, int cap,
                                               int num_ranges, int j, bool store_cu, int32_t* cu,
                                               int* s_wave_sum, int* s_start, int& c0, int& c1,
                                               int& n_chunks, ChunkPos& start) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nw = nthr / 64;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per = (B + nthr - 1) / nthr;
  const int rb = min(B, tid * per);
  const int re = min(B, rb + per);
  int local = 0;
  for (int r = rb; r < re; ++r) local += units_of<kW>(clamp_len(seq_lens[r], cap));
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave_sum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = s_wave_sum[w];
    before += w < wave ? t : 0;
    total += t;
  }
  const int excl = before + incl - local;
  if (store_cu) {
    int run = excl;
    for (int r = rb; r < re; ++r) {
      cu[r] = run;
      run += units_of<kW>(clamp_len(seq_lens[r], cap));
    }
    if (tid == 0) cu[B] = total;
  }
  const int nr = min(num_ranges, total);
  if (j >= nr) return false;   // the same for every thread of the work-group
  c0 = int(int64_t(j) * total / nr);
  c1 = int(int64_t(j + 1) * total / nr);
  int mine = 0;   // chunks of this thread's requests inside [c0, c1)
  {
    int run = excl;
    for (int r = rb; r < re; ++r) {
      const int n = units_of<kW>(clamp_len(seq_lens[r], cap));
      if (c0 >= run && c0 < run + n) {   // the request holding unit c0
        s_start[0] = r;
        s_start[1] = run + kW;
      }
      if constexpr (kW > 0) {
        if (n > 0) mine += max(0, min(c1, run + n) - max(c0, run + kW));
      }
      run += n;
    }
  }
  if constexpr (kW > 0) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o, 64);
    if (lane == 0) s_wave_sum[nw + wave] = mine;
  }
  __syncthreads();
  if constexpr (kW > 0) {
    n_chunks = 0;
    for (int w = 0; w < nw; ++w) n_chunks += s_wave_sum[nw + w];
    if (n_chunks == 0) return false;   // overhead units only (uniform)
  } else {
    n_chunks = c1 - c0;
  }
  start.r = __builtin_amdgcn_readfirstlane(s_start[0]);
  start.base = __builtin_amdgcn_readfirstlane(s_start[1]);
  start.len = clamp_len(uniform_load(seq_lens + start.r), cap);
  start.lc = max(0, c0 - start.base);
  return true;
}

}  // namespace pa
