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
// This VALU kernel serves fp32 caches; bf16 caches use the MFMA kernel below.
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
  // cache rows are read once: non-temporal loads keep them out of L2 / MALL
  __device__ __forceinline__ void stream(const uint16_t* p) { w = load16_stream(p); }
  __device__ __forceinline__ void zero() { w = u32x4_t{0, 0, 0, 0}; }
  __device__ __forceinline__ float at(int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
};
template <> struct Row8<false> {
  u32x4_t w0, w1;
  __device__ __forceinline__ void load(const float* p) { w0 = load16(p); w1 = load16(p + 4); }
  __device__ __forceinline__ void stream(const float* p) { w0 = load16_stream(p); w1 = load16_stream(p + 4); }
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
      kc[i].stream(p + (4 * i + sub) * tok_stride);
      vc[i].stream(p + kv_stride + (4 * i + sub) * tok_stride);
    }
  }
  for (; g < n_groups; g += kWaves) {
    const int gn = g + kWaves;
    if (gn < n_groups) {
      const T* p = group_ptr(gn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kn[i].stream(p + (4 * i + sub) * tok_stride);
        vn[i].stream(p + kv_stride + (4 * i + sub) * tok_stride);
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

// ---------------------------------------------------------------------------
// bf16 path on the matrix cores.  The rocprofv3 counters of the VALU kernel
// above showed it issue-bound on VALU at GQA group 8 (about 77% of the CU's
// VALU issue slots at 44% of HBM bandwidth), so for bf16 the two small
// contractions of each 32-token chunk run on v_mfma_f32_16x16x32_bf16 with
// the G query heads of the group padded to the 16 MFMA columns:
//   S^T[token][head] = K[token][:] . Q[head][:]
//   O^T[d][head]    += V^T[d][token] . P^T[token][head]
// P^T leaves the first product already in the B-operand layout of the second
// (lane l holds tokens 4(l/16)+i and 16+4(l/16)+i of head l % 16).
// Loads are fully coalesced (each instruction reads four whole 256-byte head
// rows; an operand-shaped load of sixteen 64-byte pieces measured about 15%
// less HBM bandwidth on this part) and go through a per-wave LDS tile that
// is read back in operand order: K rows with ds_read_b128, V^T with
// ds_read_b64_tr_b16.  16-byte chunk c of token row t sits in LDS slot
// c ^ (t % 16), so both the row writes and the column reads are spread over
// all banks.  Lanes l, l^16, l^32, l^48 hold the four token slices of head
// l % 16.  One register set per wave and no software prefetch: at three
// waves per SIMD nearly every wave's buffers are waiting on HBM at any time.
constexpr int kChunk = 32;                 // tokens per MFMA chunk
constexpr int kTileRow = kD * 2;           // LDS row of one token (256 B)

// Byte offset of 16-byte chunk c of token row t in a swizzled tile.
__device__ __forceinline__ int tile_off(int t, int c) { return t * kTileRow + 16 * (c ^ (t & 15)); }

template <int G>
__global__ __launch_bounds__(256, 4) void decode_mfma_kernel(DecodeGQA a) {
  static_assert(G >= 1 && G <= 16, "group must fit the 16 MFMA columns");
  // per-wave tile (K, then V of the same chunk); reused for the final merge
  constexpr int kTileBytes = kChunk * kTileRow;
  constexpr int kMergeBytes = kWaves * G * (kD + 2) * 4;
  constexpr int kSmem = kWaves * kTileBytes > kMergeBytes ? kWaves * kTileBytes : kMergeBytes;
  __shared__ __align__(16) char smem[kSmem];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int li = lane & 15;   // token (A operand) / head (B operand) index
  const int kq = lane >> 4;   // 16-lane group

  const int Hkv = a.num_kv_heads;
  const int S = a.num_splits;
  int id = blockIdx.x;
  const int h = id % Hkv; id /= Hkv;
  const int s = id % S;
  const int r = id / S;
  const int Hq = a.num_q_heads;
  const int bs = a.block_size;
  const int seq = min(a.seq_lens[r], a.max_blocks * bs);
  const int t0 = s * a.split_tokens;
  if (t0 >= seq) {
    if (!a.direct && threadIdx.x < G)
      a.part[((int64_t(r) * Hq + int64_t(h) * G + threadIdx.x) * S + s) * (kD + 1) + kD] = -INFINITY;
    if (a.direct) {
      for (int i = threadIdx.x; i < G * kD; i += blockDim.x)
        static_cast<uint16_t*>(a.out)[(int64_t(r) * Hq + int64_t(h) * G) * kD + i] = 0;
      if (a.lse && threadIdx.x < G) a.lse[int64_t(r) * Hq + int64_t(h) * G + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int t1 = min(seq, t0 + a.split_tokens);
  const int n_chunks = (t1 - t0 + kChunk - 1) / kChunk;
  const float scale2 = a.scale * kLog2e;
  const int64_t tok_stride = int64_t(Hkv) * kD;
  const int64_t kv_stride = int64_t(bs) * tok_stride;
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache);
  const int32_t* table = a.block_table + int64_t(r) * a.max_blocks;

  // Q^T (B operand): head li of the group, dims 32 kk + 8 kq .. + 8; zero past G
  u32x4_t qf[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (int64_t(r) * Hq + int64_t(h) * G + (li < G ? li : 0)) * kD + 8 * kq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = li < G ? load16(qp + 32 * kk) : u32x4_t{0, 0, 0, 0};
  }

  // Coalesced K/V loads of a chunk: instruction i reads tokens 4i + (l / 16),
  // lane l taking 16-byte chunk l % 16 of the head row.  Tokens past the split
  // end re-read its last token (finite data, masked out below); the loads are
  // unconditional so the vector-memory waits stay exact.
  const int lc = lane & 15;   // chunk of the head row this lane loads
  const int lt = lane >> 4;   // token within a 4-token load
  const int last16 = ((t1 - 1) / 16) * 16;
  auto load_chunk = [&](int c, u32x4_t (&kr)[8], u32x4_t (&vr)[8]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int tok16 = min(t0 + c * kChunk + 16 * sub, last16);
      int64_t blk = uniform_load(table + tok16 / bs);
      blk = (blk < 0 || blk >= a.num_blocks) ? 0 : blk;
      const int page0 = (tok16 / bs) * bs;     // first token of the page
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = min(tok16 + 4 * i + lt, t1 - 1);
        const int64_t off = (blk * 2 * bs + (tok - page0)) * tok_stride + int64_t(h) * kD + 8 * lc;
        kr[4 * sub + i] = load16_stream(cache + off);
        vr[4 * sub + i] = load16_stream(cache + off + kv_stride);
      }
    }
  };

  f32x4_t acc[8];   // O^T: d = 16 dt + 4 kq + i, head li
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0, 0, 0, 0};
  float m_run = kNoMax, l_run = 0.0f;
  char* tl = smem + wave * kTileBytes;

  for (int c = wave; c < n_chunks; c += kWaves) {
    u32x4_t kr[8], vr[8];
    load_chunk(c, kr, vr);
    // K rows into the tile, then read back as A operands (token li of each
    // 16-token half, dims 32 kk + 8 kq)
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(tl + tile_off(4 * i + lt, lc)) = kr[i];
    f32x4_t sc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sc[sub] = f32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(tl + tile_off(16 * sub + li, 4 * kk + kq));
        sc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[kk]), sc[sub], 0, 0, 0);
      }
    }
    // V rows into the same tile (this wave's LDS operations execute in order,
    // and the K reads above have been consumed by the MFMAs)
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(tl + tile_off(4 * i + lt, lc)) = vr[i];

    const int tokc = t0 + c * kChunk;
    const bool tail = tokc + kChunk > t1;
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sc[sub][i] * scale2;
        if (tail && tokc + 16 * sub + 4 * kq + i >= t1) v = -INFINITY;
        sc[sub][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, lane_xor(tmax, 16));
    tmax = fmaxf(tmax, lane_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float p[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(sc[0][i] - m_new);
      p[4 + i] = fast_exp2(sc[1][i] - m_new);
      psum += p[i] + p[4 + i];
    }
    l_run = fmaf(l_run, alpha, psum);
    const u32x4_t pf = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                               pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    // O^T += V^T P^T.  Lane gi of 16-lane group kq reads 4 bf16 of token row
    // 4 kq + gi/4 (+16) at dims 16 dt + 4 (gi % 4): chunk 2 dt + (gi % 4)/2.
    const int vrow = 4 * kq + (li >> 2);
    const int vhalf = 8 * (li & 1);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int ch = 2 * dt + ((li & 3) >> 1);
      const uint2 v1 = lds_read_tr(tl + tile_off(vrow, ch) + vhalf);
      const uint2 v2 = lds_read_tr(tl + tile_off(vrow + 16, ch) + vhalf);
      acc[dt] *= alpha;
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          as_bf16x8(u32x4_t{v1.x, v1.y, v2.x, v2.y}), as_bf16x8(pf), acc[dt], 0, 0, 0);
    }
  }

  // this wave's state for head li: sum l over the four token slices
  const float l_w = l_run + lane_xor(l_run, 16);
  const float l_tot = l_w + lane_xor(l_w, 32);
  __syncthreads();   // every wave is done with its tile: reuse the LDS for the merge
  float* s_acc = reinterpret_cast<float*>(smem);                 // [wave][G][kD]
  float* s_ml = s_acc + kWaves * G * kD;                         // [wave][G][2]
  if (li < G) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_acc[(wave * G + li) * kD + 16 * dt + 4 * kq + i] = acc[dt][i];
    if (kq == 0) { s_ml[(wave * G + li) * 2] = m_run; s_ml[(wave * G + li) * 2 + 1] = l_tot; }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += blockDim.x) {
    const int j = idx / kD;
    const int d = idx - j * kD;
    float mm = s_ml[j * 2];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, s_ml[(w * G + j) * 2]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_ml[(w * G + j) * 2] - mm);
      num = fmaf(f, s_acc[(w * G + j) * kD + d], num);
      den = fmaf(f, s_ml[(w * G + j) * 2 + 1], den);
    }
    const float o = num / den;
    const int64_t row = int64_t(r) * Hq + int64_t(h) * G + j;
    if (a.direct) {
      static_cast<uint16_t*>(a.out)[row * kD + d] = f32_to_bf16(o);
      if (d == 0 && a.lse) a.lse[row] = (mm + fast_log2(den)) * kLn2;
    } else {
      float* pp = a.part + (row * S + s) * (kD + 1);
      pp[d] = o;
      if (d == 0) pp[kD] = (mm + fast_log2(den)) * kLn2;
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

template <int kPer>   // dims per lane: ceil(Dv / 64)
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
    // splits wave, wave + 4, ...: eight rows in flight per step; empty splits
    // (weight 0) are skipped by a select, not a branch, so loads pipeline
    int s0 = wave;
    for (; s0 + 28 < cn; s0 += 32) {
      float w[8];
      float v[8][kPer];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        w[u] = s_w[s0 + 4 * u];
        const float* row = base + (c0 + s0 + 4 * u) * stride;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int d = lane + 64 * i;
          v[u][i] = d < Dv ? row[d] : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] += w[u] != 0.0f ? w[u] * v[u][i] : 0.0f;
    }
    for (; s0 < cn; s0 += 4) {
      const float w = s_w[s0];
      const float* row = base + (c0 + s0) * stride;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int d = lane + 64 * i;
        const float x = d < Dv ? row[d] : 0.0f;
        acc[i] += w != 0.0f ? w * x : 0.0f;
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

hipError_t launch_decode_bf16(const DecodeGQA& a, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_kv_heads * a.num_splits)), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_mfma_kernel<1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_mfma_kernel<2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeGQA& a, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_kv_heads * a.num_splits)), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<false, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<false, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<false, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<false, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gqa(const DecodeGQA& a, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  return a.bf16 ? launch_decode_bf16(a, s) : launch_decode_f32(a, s);
}

hipError_t launch_lse_merge(const LseMerge& a, hipStream_t s) {
  const int64_t pairs = int64_t(a.num_rows) * a.num_heads;
  if (pairs <= 0) return hipSuccess;
  if (a.head_dim_v > kMergeMaxDv || pairs > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid{unsigned(pairs)}, block{unsigned(kMergeThreads)};
  if (a.head_dim_v <= 128) hipLaunchKernelGGL(lse_merge_kernel<2>, grid, block, 0, s, a);
  else if (a.head_dim_v <= 512) hipLaunchKernelGGL(lse_merge_kernel<8>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(lse_merge_kernel<16>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
