// Varlen causal prefill / chunked-prefill extend over the paged cache.
//
// Method: "第 1 章 注意力后端" §4.1 (FlashAttention-style tiling: bring a
// block of K/V on chip, compute that block's scores, update the running max
// and normaliser, rescale the accumulated output, never materialise the
// score matrix) with the causal mask of §2.1, bottom-right aligned for a
// chunk of L new queries over S keys (query i sees keys j <= S - L + i).
// Requests are delimited by query_start_loc and seq_lens; keys are gathered
// through block_table ("Attention Backends", step 2).
//
// gfx950 mapping.  A work-group of 4 waves owns 128 query rows of one query
// head of one request; wave w owns rows 32w..32w+31.  K/V tiles of 64 keys
// are gathered from their pages into LDS (double-buffered, rows padded to
// 272 B) by all 256 threads.  Both products run on v_mfma_f32_32x32x16_bf16
// in transposed form so that each lane owns one query row:
//   S^T[key][row] = K[key][:] . Q[row][:]     A = K rows (LDS), B = Q (regs)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  A = V^T (LDS transpose
//                   reads, ds_read_b64_tr_b16), B = P^T (the S^T registers)
// With the MFMA output layout (lane l holds column l % 32) the row max,
// running sum and rescale of a query row live in lane l and lane l ^ 32.
// Tiles entirely above the diagonal are skipped; diagonal tiles mask per
// element.  Work-groups are ordered longest tile first.
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kBM = 128;           // query rows per work-group
constexpr int kBN = 64;            // keys per tile
constexpr int kRowBytes = kD * 2 + 16;   // padded LDS row (bank spread)
constexpr int kTileBytes = kBN * kRowBytes;

typedef __attribute__((ext_vector_type(4))) short s16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Four b16 values from LDS, transposed within each 16-lane group: lane i of
// the group receives element (i % 4) of the 8-byte chunks addressed by lanes
// 4q + i/4, q = 0..3 (so a group reading a 4-row x 16-column block gets one
// column of 4 rows per lane).
__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s4;
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
  return __builtin_bit_cast(uint2, v);
}

__global__ __launch_bounds__(256) void prefill_kernel(PrefillVarlen a) {
  __shared__ __align__(16) char smem[4 * kTileBytes];   // 2 x (K tile, V tile)
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int tid = threadIdx.x;
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;

  // work-group -> (q tile, request, head); larger tile index first
  const int n_qt = (a.max_query_len + kBM - 1) / kBM;
  int id = blockIdx.x;
  const int h = id % Hq; id /= Hq;
  const int r = id % a.num_seqs;
  const int qt = n_qt - 1 - id / a.num_seqs;
  const int q_start = min(max(a.query_start_loc[r], 0), a.num_tokens);
  const int L = min(min(a.query_start_loc[r + 1] - q_start, a.max_query_len), a.num_tokens - q_start);
  const int bs = a.block_size;
  const int S = min(a.seq_lens[r], a.max_blocks * bs);
  const int q0 = qt * kBM;
  if (q0 >= L || L <= 0) return;
  const int C = S - L;                    // keys before the chunk
  const int kvh = h / G;

  // keys this work-group may see
  int kv_end = S;
  if (a.causal) kv_end = min(S, max(0, C + min(q0 + kBM, L)));
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // ---- Q fragments (B operand of S^T): row = l % 32, d chunk = 16 kk + 8 (l / 32)
  const int my_row = q0 + wave * 32 + (lane & 31);
  const bool row_ok = my_row < L;
  u32x4_t qf[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (int64_t(q_start) + (row_ok ? my_row : 0)) * Hq * kD + int64_t(h) * kD +
                         8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = row_ok ? load16(qp + 16 * kk) : u32x4_t{0, 0, 0, 0};
  }

  // ---- cooperative gather of one K/V tile: 64 keys x 16 chunks of 16 B each
  const int64_t tok_stride = int64_t(a.num_kv_heads) * kD;
  const int64_t kv_stride = int64_t(bs) * tok_stride;
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache);
  const int32_t* table = a.block_table + int64_t(r) * a.max_blocks;
  const int ld_chunk = tid & 15;
  const int ld_key = tid >> 4;           // + 16 i, i = 0..3
  u32x4_t stk[4], stv[4];
  // Keys ld_key + 16 i of a tile share one page per i (tiles and 16-key groups
  // are 16-aligned, pages are multiples of 16): the page ids are wave-uniform
  // scalar loads.  Keys past kv_end re-read key kv_end - 1 (finite, masked
  // out below), so every load is unconditional and the waits stay exact.
  auto gload = [&](int tile) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key16 = min(tile * kBN + 16 * i, ((kv_end - 1) / 16) * 16);
      int64_t blk = uniform_load(table + key16 / bs);
      blk = (blk < 0 || blk >= a.num_blocks) ? 0 : blk;
      const int key = min(key16 + ld_key, kv_end - 1);
      const uint16_t* p = cache + (blk * 2 * bs + (key - (key16 / bs) * bs)) * tok_stride +
                          int64_t(kvh) * kD + 8 * ld_chunk;
      stk[i] = load16(p);
      stv[i] = load16(p + kv_stride);
    }
  };
  auto lstore = [&](int buf) {
    char* kt = smem + buf * 2 * kTileBytes;
    char* vt = kt + kTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = (ld_key + 16 * i) * kRowBytes + ld_chunk * 16;
      *reinterpret_cast<u32x4_t*>(kt + off) = stk[i];
      *reinterpret_cast<u32x4_t*>(vt + off) = stv[i];
    }
  };

  const float scale2 = a.scale * kLog2e;
  float m_run = kNoMax;   // running max (base-2 domain) of row my_row
  float l_run = 0.0f;     // this lane's share of the running sum
  f32x16_t acc[4];        // O^T tiles: d = 32 dt + 8 (r/4) + 4 (l/32) + r%4
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;

  if (n_tiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  const int row_abs = C + my_row;         // last key this row may see (causal)
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);    // in flight during the math below
    const char* kt = smem + buf * 2 * kTileBytes;
    const char* vt = kt + kTileBytes;
    const int key0 = t * kBN;

    // S^T for two 32-key halves
    f32x16_t s[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[hh][i] = 0.0f;
      const char* krow = kt + (hh * 32 + (lane & 31)) * kRowBytes + 16 * (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(krow + 32 * kk);
        s[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[kk]), s[hh], 0, 0, 0);
      }
    }

    // mask, scale, tile max (keys of this lane, then lane ^ 32)
    const bool need_mask = (key0 + kBN > kv_end) || (a.causal && key0 + kBN - 1 > C + q0 + wave * 32);
    float tmax = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[hh][i] * scale2;
        if (need_mask) {
          const int key = key0 + hh * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          const bool vis = key < kv_end && (!a.causal || key <= row_abs);
          v = vis ? v : -INFINITY;
        }
        s[hh][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, lane_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    // P^T in bf16, packed as the B operand: regs 8 st .. 8 st + 7 of half hh
    u32x4_t pf[4];
    float psum = 0.0f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(s[hh][8 * st + j] - m_new);
          psum += p[j];
        }
        pf[2 * hh + st] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                  pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;

    // O^T += V^T P^T: 4 key steps of 16 x 4 d tiles of 32
    const int grp = lane >> 4;              // 16-lane group
    const int gi = lane & 15;
    const int kg = lane >> 5;               // k group
    const int dhalf = grp & 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kbase = 16 * ks + 4 * kg;   // keys kbase..+3 and kbase+8..+11
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dcol = 32 * dt + 16 * dhalf + 4 * (gi & 3);
        const uint32_t o1 = uint32_t((kbase + (gi >> 2)) * kRowBytes + dcol * 2);
        const uint32_t o2 = o1 + 8 * kRowBytes;
        const uint2 v1 = lds_read_tr(vt + o1);
        const uint2 v2 = lds_read_tr(vt + o2);
        const u32x4_t vf = u32x4_t{v1.x, v1.y, v2.x, v2.y};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), acc[dt], 0, 0, 0);
      }
    }

    if (t + 1 < n_tiles) {
      // buffer buf ^ 1 was last read in iteration t - 1, which every wave
      // finished before the barrier that ended it
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- finish: full row sum, normalise, write
  const float l_tot = l_run + lane_xor(l_run, 32);
  if (!row_ok) return;
  const int64_t orow = int64_t(q_start) + my_row;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* op = static_cast<uint16_t*>(a.out) + orow * Hq * kD + int64_t(h) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * dt + 8 * q4 + 4 * (lane >> 5);
      uint2 w;
      w.x = pack_bf16x2(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv);
      w.y = pack_bf16x2(acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = w;
    }
  if (a.lse && lane < 32)
    a.lse[orow * Hq + h] = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_varlen(const PrefillVarlen& a, hipStream_t s) {
  if (a.num_seqs <= 0 || a.num_tokens <= 0 || a.max_query_len <= 0) return hipSuccess;
  const int n_qt = (a.max_query_len + kBM - 1) / kBM;
  const int64_t wgs = int64_t(n_qt) * a.num_seqs * a.num_q_heads;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_kernel, dim3(unsigned(wgs)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
