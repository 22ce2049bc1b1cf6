// MLA decode over the latent cache, split-KV partials merged by LSE.
//
// Method: "Triton 與 MLA：可移植注意力與潛空間注意力" (設計動機, 資料流): the cache
// holds one row [kv_c (512) | k_pe (64)] per token, read as a single key
// head shared by every query head (MQA); the query is [q_nope | q_pe]; the
// value is the first 512 columns of the same row; partial outputs of each KV
// split carry their lse for the stage-2 merge.  Online softmax as in
// "第 1 章 注意力后端" §4.1.
//
// gfx950 mapping.  One work-group of 8 waves owns (request, split) for all
// H <= 128 query heads; wave w owns heads 16w..16w+15 (waves past H/16 only
// help gather tiles).  Because every head reads the
// same latent row, the work is a real dense contraction: per 32-key tile,
// S^T[32 keys x 16 heads] = K[32 x 576] Q^T[576 x 16] (18 k-steps of
// v_mfma_f32_16x16x32_bf16 per 16 keys) and O^T[512 x 16] += V^T[512 x 32]
// P^T[32 x 16] (32 MFMAs, V^T read with ds_read_b64_tr_b16).  Each latent
// row is fetched from HBM once per work-group into a double-buffered LDS tile
// and feeds both products.  Lanes l, l^16, l^32, l^48 share head l % 16; the
// per-head softmax state lives there.
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kRank = 512;
constexpr int kRope = 64;
constexpr int kRow = kRank + kRope;             // 576 elements
constexpr int kChunks = kRow * 2 / 16;          // 72 x 16 B per row
constexpr int kBN = 32;                         // keys per tile
constexpr int kRowBytes = kRow * 2;             // 1152 B, unpadded (swizzled)
constexpr int kTileBytes = kBN * kRowBytes;     // 36864 B
constexpr int kTileLoads = kBN * kChunks / 64;  // 36 wave-wide 16-byte loads per tile
constexpr int kMaxWaves = 8;

// 16-byte chunk c of latent row r sits in LDS slot c ^ (r % 8) of the row
// (within its aligned group of eight), spreading K-row and V-column reads
// over all banks.
__device__ __forceinline__ int tile_off(int r, int c) { return r * kRowBytes + 16 * (c ^ (r & 7)); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (one head).
__device__ __forceinline__ float head_max(float x) {
  x = fmaxf(x, lane_xor(x, 16));
  return fmaxf(x, lane_xor(x, 32));
}
__device__ __forceinline__ float head_sum(float x) {
  x += lane_xor(x, 16);
  return x + lane_xor(x, 32);
}

__global__ __launch_bounds__(512) void mla_split_kernel(MlaDecode a) {
  __shared__ __align__(16) char smem[2 * kTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nthreads = blockDim.x;
  const int tid = threadIdx.x;
  const int H = a.num_heads;

  const int S_spl = a.num_splits;
  const int s = blockIdx.x % S_spl;
  const int r = blockIdx.x / S_spl;
  const int bs = a.block_size;
  const int seq = min(a.seq_lens[r], a.max_blocks * bs);
  const int t0 = s * a.split_tokens;
  if (t0 >= seq) {   // empty split: weight 0 in the merge (direct: no key at all)
    for (int hd = tid; hd < H; hd += nthreads) {
      const int64_t row = int64_t(r) * H + hd;
      if (!a.direct) {
        a.part[(row * S_spl + s) * (kRank + 1) + kRank] = -INFINITY;
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out) + row * kRank;
        for (int d = 0; d < kRank; ++d) op[d] = 0;
        if (a.lse) a.lse[row] = -INFINITY;
      }
    }
    return;
  }
  const int t1 = min(seq, t0 + a.split_tokens);
  const int n_tiles = (t1 - t0 + kBN - 1) / kBN;

  // ---- Q^T fragments: head = 16 wave + l % 16, dims 32 kk + 8 (l / 16) .. + 8
  const bool active = wave < H / 16;
  const int head = active ? 16 * wave + (lane & 15) : 0;
  const int kq = lane >> 4;
  u32x4_t qf[18];
  {
    const uint16_t* qn = static_cast<const uint16_t*>(a.q_nope) + int64_t(r) * a.qn_sb +
                         int64_t(head) * a.qn_sh;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_pe) + int64_t(r) * a.qp_sb +
                         int64_t(head) * a.qp_sh;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk] = load16(qn + 32 * kk + 8 * kq);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qf[16 + kk] = load16(qp + 32 * kk + 8 * kq);
  }

  // ---- gather of a tile straight into LDS: 36 wave-wide loads of 64 x 16 B
  // (global_load_lds_dwordx4; lane i lands at byte 16 i of the load's 1 KiB),
  // wave w issuing loads w, w + 8, ...  Position p = 64 j + i of load j is
  // row p / 72, slot p % 72, which holds chunk slot ^ (row % 8).  A 32-key
  // tile spans at most two pages, whose ids are wave-uniform scalar loads.
  // Keys past t1 re-read key t1 - 1 (finite, masked out below).
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache);
  const int32_t* table = a.block_table + int64_t(r) * a.max_blocks;
  auto gload = [&](int tile, char* dst) {
    const int key0 = t0 + tile * kBN;
    const int kl0 = min(key0, t1 - 1), kl1 = min(key0 + kBN - 1, t1 - 1);
    int64_t b0 = uniform_load(table + kl0 / bs), b1 = uniform_load(table + kl1 / bs);
    b0 = (b0 < 0 || b0 >= a.num_blocks) ? 0 : b0;
    b1 = (b1 < 0 || b1 >= a.num_blocks) ? 0 : b1;
    const int pg0 = kl0 / bs;
    for (int j = wave; j < kTileLoads; j += kMaxWaves) {
      const int pos = 64 * j + lane;
      const int row = pos / kChunks;
      const int slot = pos - row * kChunks;
      const int key = min(key0 + row, t1 - 1);
      const int64_t blk = (key / bs == pg0) ? b0 : b1;
      const uint16_t* src = cache + (blk * bs + (key % bs)) * kRow + 8 * (slot ^ (row & 7));
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + 1024 * j),
                                       16, 0, 0);
    }
  };
  // all of this wave's tile loads have landed (the caller then syncs the group)
  auto gwait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  const float scale2 = a.scale * kLog2e;
  float m_run = kNoMax;
  float l_run = 0.0f;          // this lane's share of head `head`'s sum
  f32x4_t acc[32];             // O^T: d = 16 dt + 4 (l / 16) + r
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0, 0, 0, 0};

  gload(0, smem);
  gwait();
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1, smem + (buf ^ 1) * kTileBytes);
    const char* tl = smem + buf * kTileBytes;
    const int key0 = t0 + t * kBN;
    if (active) {
    // S^T halves: keys 16 hh + 4 (l/16) + r, head l % 16
    f32x4_t sc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      sc[hh] = f32x4_t{0, 0, 0, 0};
      // chunk 4 kk + kq of row krow: slot 8 (kk / 2) + ((4 (kk % 2) + kq) ^ (krow % 8)),
      // i.e. two per-lane bases plus a constant offset per kk
      const int krow = 16 * hh + (lane & 15);
      const char* kb0 = tl + krow * kRowBytes + 16 * (kq ^ (krow & 7));
      const char* kb1 = tl + krow * kRowBytes + 16 * ((4 + kq) ^ (krow & 7));
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>((kk & 1 ? kb1 : kb0) + 128 * (kk >> 1));
        sc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[kk]), sc[hh], 0, 0, 0);
      }
    }
    const bool tail = key0 + kBN > t1;
    float tmax = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sc[hh][i] * scale2;
        if (tail && key0 + 16 * hh + 4 * kq + i >= t1) v = -INFINITY;
        sc[hh][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = head_max(tmax);
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
    l_run = l_run * alpha + psum;
    const u32x4_t pf = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                               pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    // O^T += V^T P^T: keys 4 kq + (0..3) and 16 + 4 kq + (0..3)
    // lane gi of group kq: 4 bf16 of rows 4 kq + gi/4 (+16) at dims
    // 16 dt + 4 (gi % 4), i.e. chunk 2 dt + (gi % 4)/2, half gi % 2
    // (slot 8 (dt / 4) + ((2 (dt % 4) + (gi % 4)/2) ^ (row % 8)): four per-lane
    // bases plus a constant offset per dt; rows vrow and vrow + 16 share row % 8)
    const int gi = lane & 15;
    const int vrow = 4 * kq + (gi >> 2);
    const int bsel = (gi & 3) >> 1;
    const char* vb[4];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4)
      vb[m4] = tl + vrow * kRowBytes + 16 * ((2 * m4 + bsel) ^ (vrow & 7)) + 8 * (gi & 1);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const char* vp = vb[dt & 3] + 128 * (dt >> 2);
      const uint2 v1 = lds_read_tr(vp);
      const uint2 v2 = lds_read_tr(vp + 16 * kRowBytes);
      const u32x4_t vf = u32x4_t{v1.x, v1.y, v2.x, v2.y};
      acc[dt] *= alpha;
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), as_bf16x8(pf), acc[dt], 0, 0, 0);
    }
    }  // active
    if (t + 1 < n_tiles) {
      gwait();           // this wave's loads of tile t + 1 have landed
      __syncthreads();   // everyone's have, and everyone is done with tile t
    }
  }

  // ---- finish: per-head sum over the 4 lanes, normalise, write
  if (!active) return;
  const float l_tot = head_sum(l_run);
  const float inv = 1.0f / l_tot;
  const float lse_nat = (m_run + fast_log2(l_tot)) * kLn2;
  const int64_t row = int64_t(r) * H + head;
  if (a.direct) {
    uint16_t* op = static_cast<uint16_t*>(a.out) + row * kRank;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      w.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * dt + 4 * kq) = w;
    }
    if (kq == 0 && a.lse) a.lse[row] = lse_nat;
  } else {
    float* pp = a.part + (row * S_spl + s) * (kRank + 1);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[16 * dt + 4 * kq + i] = acc[dt][i] * inv;
    if (kq == 0) pp[kRank] = lse_nat;
  }
}

}  // namespace

hipError_t launch_mla_decode(const MlaDecode& a, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  if (a.rank != kRank || a.rope != kRope || a.num_heads % 16 || a.num_heads > 16 * kMaxWaves)
    return hipErrorNotSupported;
  const int64_t wgs = int64_t(a.num_seqs) * a.num_splits;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_split_kernel, dim3(unsigned(wgs)), dim3(64 * kMaxWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
