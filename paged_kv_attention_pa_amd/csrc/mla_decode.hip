// MLA decode over the latent cache, split-KV partials merged by LSE.
//
// Method: "Triton 與 MLA：可移植注意力與潛空間注意力" (設計動機, 資料流): the cache
// holds one row [kv_c (512) | k_pe (64)] per token, read as a single key
// head shared by every query head (MQA); the query is [q_nope | q_pe]; the
// value is the first 512 columns of the same row; partial outputs of each KV
// split carry their lse for the stage-2 merge.  Online softmax as in
// "第 1 章 注意力后端" §4.1.
//
// gfx950 mapping.  One work-group of 8 waves owns a run of 32-key tiles for
// all H <= 128 query heads; wave w owns heads 16w..16w+15 (waves past H/16
// only help gather tiles).  Because every head reads the same latent row, the
// work is a real dense contraction: per tile, S^T[32 keys x 16 heads] =
// K[32 x 576] Q^T[576 x 16] (18 k-steps of v_mfma_f32_16x16x32_bf16 per 16
// keys) and O^T[512 x 16] += V^T[512 x 32] P^T[32 x 16] (32 MFMAs, V^T read
// with ds_read_b64_tr_b16).  Each latent row is fetched from HBM once per
// work-group into an LDS tile (global_load_lds_dwordx4, swizzled, two
// buffers) and feeds both products.  Lanes l, l^16, l^32, l^48 share head
// l % 16; the per-head softmax state lives there, and the running max is
// rescaled lazily (only when a head's max grows by more than kSlack).
// The LDS reads of a tile are issued as inline assembly and waited for
// explicitly: the compiler would otherwise wait for the next tile's loads,
// still in flight, before reading the current one (it cannot tell the two
// buffers apart), which serialises the pipeline.
#include "balanced.hpp"
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
constexpr int kStages = 2;                      // LDS tile buffers: kStages - 1 tiles in flight
constexpr float kSlack = 8.0f;                  // lazy-rescale headroom, log2 units

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

// Two schedules share the kernel body:
// * kBalanced = false: work-group (request, split) over keys [t0, t1) of one
//   request, split s = [s P, (s+1) P); partials [B, H, S, 513] for the merge.
// * kBalanced = true: work-group j walks chunk range j of the batch's chunk
//   list (balanced.hpp), finishing the requests inside it and leaving segment
//   partials [(nr + B) H, 516] for the others.
// A "tile" is 32 keys [kb + 32 lc, kb + 32 lc + 32) of request r, keys at or
// past kend masked (split: kb = t0, kend = t1; balanced: kb = 0, kend = len).
template <bool kBalanced>
__global__ __launch_bounds__(512) void mla_kernel(MlaDecode a) {
  __shared__ __align__(16) char smem[kStages * kTileBytes];
  __shared__ int s_wave_sum[kMaxWaves];
  __shared__ int s_start[2];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int tid = threadIdx.x;
  const int H = a.num_heads;
  const int B = a.num_seqs;
  const int bs = a.block_size;
  const int cap = a.max_blocks * bs;

  // ---- this work-group's tiles
  int j = 0, s = 0, n_tiles = 0, c0 = 0, c1 = 0, kb = 0;
  ChunkPos cur;   // r, lc (tile index), kend, base (list index of the request's first chunk)
  if constexpr (kBalanced) {
    j = blockIdx.x;
    if (!balanced_range(a.seq_lens, B, cap, a.num_ranges, j, j == 0, a.cu, s_wave_sum, s_start,
                        c0, c1, cur))
      return;
    n_tiles = c1 - c0;
  } else {
    const int S_spl = a.num_splits;
    s = blockIdx.x % S_spl;
    const int r = blockIdx.x / S_spl;
    const int seq = min(a.seq_lens[r], cap);
    const int t0 = s * a.split_tokens;
    if (t0 >= seq) {   // empty split: weight 0 in the merge (direct: no key at all)
      for (int hd = tid; hd < H; hd += blockDim.x) {
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
    n_tiles = (t1 - t0 + kBN - 1) / kBN;
    kb = t0;
    cur = ChunkPos{r, 0, t1, 0};
  }
  auto advance = [&](const ChunkPos& p) {
    if constexpr (kBalanced) {
      return next_chunk(p, a.seq_lens, cap, B);
    } else {
      return ChunkPos{p.r, p.lc + 1, p.len, p.base};
    }
  };

  // ---- Q^T fragments: head = 16 wave + l % 16, dims 32 kk + 8 (l / 16) .. + 8
  const bool active = wave < H / 16;
  const int head = active ? 16 * wave + (lane & 15) : 0;
  const int kq = lane >> 4;
  u32x4_t qf[18];
  auto load_q = [&](int r) {
    const uint16_t* qn = static_cast<const uint16_t*>(a.q_nope) + int64_t(r) * a.qn_sb +
                         int64_t(head) * a.qn_sh;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_pe) + int64_t(r) * a.qp_sb +
                         int64_t(head) * a.qp_sh;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk] = load16(qn + 32 * kk + 8 * kq);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qf[16 + kk] = load16(qp + 32 * kk + 8 * kq);
  };

  // ---- gather of a tile straight into LDS: 36 wave-wide loads of 64 x 16 B
  // (global_load_lds_dwordx4; lane i lands at byte 16 i of the load's 1 KiB),
  // wave w issuing loads w, w + 8, ...  Position p = 64 j + i of load j is
  // row p / 72, slot p % 72, which holds chunk slot ^ (row % 8).  A 32-key
  // tile spans at most two pages, whose ids are wave-uniform scalar loads.
  // Keys at or past kend re-read key kend - 1 (finite, masked out below).
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache);
  auto gload = [&](const ChunkPos& p, char* dst) {
    const int32_t* table = a.block_table + int64_t(p.r) * a.max_blocks;
    const int key0 = kb + p.lc * kBN;
    const int kend = p.len;
    const int kl0 = min(key0, kend - 1), kl1 = min(key0 + kBN - 1, kend - 1);
    int64_t b0 = uniform_load(table + kl0 / bs), b1 = uniform_load(table + kl1 / bs);
    b0 = (b0 < 0 || b0 >= a.num_blocks) ? 0 : b0;
    b1 = (b1 < 0 || b1 >= a.num_blocks) ? 0 : b1;
    // key0 + row sits at offset kin = (key0 % bs) + row of page b0, or
    // kin - bs of page b1 (key0 is a multiple of 16 below one page's end)
    const int in0 = key0 % bs;
    const int last = kend - 1 - key0 + in0;          // offset of key kend - 1
    const int64_t o0 = b0 * bs * kRow, o1 = (b1 - 1) * bs * kRow;
    for (int jl = wave; jl < kTileLoads; jl += kMaxWaves) {
      const int pos = 64 * jl + lane;
      const int row = pos / kChunks;
      const int slot = pos - row * kChunks;
      const int kin = min(in0 + row, last);
      const uint16_t* src = cache + ((kin < bs ? o0 : o1) + kin * kRow + 8 * (slot ^ (row & 7)));
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + 1024 * jl),
                                       16, 0, 0);
    }
  };
  // all of this wave's loads have landed (the caller then syncs the group)
  auto gwait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  const float scale2 = a.scale * kLog2e;
  float m_run = kNoMax;
  float l_run = 0.0f;          // this lane's share of head `head`'s sum
  f32x4_t acc[32];             // O^T: d = 16 dt + 4 (l / 16) + r
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0, 0, 0, 0};

  // ---- finish a segment: per-head sum over the 4 lanes, normalise, write
  auto finish = [&](const ChunkPos& p) {
    const float l_tot = head_sum(l_run);
    if (!active) return;
    const float inv = 1.0f / l_tot;
    const float lse_nat = (m_run + fast_log2(l_tot)) * kLn2;
    const int64_t row = int64_t(p.r) * H + head;
    bool direct;
    float* pp;
    if constexpr (kBalanced) {
      direct = p.base >= c0 && p.base + chunks_of(p.len) <= c1;
      pp = a.part + (int64_t(j + p.r) * H + head) * (kRank + 4);
    } else {
      direct = a.direct;
      pp = a.part + (row * a.num_splits + s) * (kRank + 1);
    }
    if (direct) {
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
#pragma unroll
      for (int dt = 0; dt < 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pp[16 * dt + 4 * kq + i] = acc[dt][i] * inv;
      if (kq == 0) pp[kRank] = lse_nat;
    }
  };

  // Tile pipeline: kStages - 1 tiles are loading while one is computed.  Each
  // wave issues n_w of a tile's loads (36 over 8 waves: 5 or 4), so "tile t
  // has landed" is "at most n_w x (tiles issued after t) loads outstanding".
  const int n_w = (kTileLoads + kMaxWaves - 1 - wave) / kMaxWaves;
  auto wait_tiles = [&](int k) {   // k = tiles issued after the one waited for, <= kStages - 2
    if (n_w == 5) {
      if (k <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
      else if (k == 1) __builtin_amdgcn_s_waitcnt(0x0F75);   // vmcnt(5)
      else __builtin_amdgcn_s_waitcnt(0x0F7A);               // vmcnt(10)
    } else {
      if (k <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
      else if (k == 1) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
      else __builtin_amdgcn_s_waitcnt(0x0F78);               // vmcnt(8)
    }
  };
  static_assert(kStages >= 2 && kStages <= 4 && kTileLoads == 36 && kMaxWaves == 8,
                "wait_tiles counts");

  load_q(cur.r);
  gwait();   // q is in registers before any tile load is issued
  ChunkPos ld = cur;   // next tile to load
  int n_loaded = 0;
  for (; n_loaded < kStages - 1 && n_loaded < n_tiles; ++n_loaded) {
    gload(ld, smem + n_loaded * kTileBytes);
    if (n_loaded + 1 < n_tiles) ld = advance(ld);
  }

  for (int t = 0; t < n_tiles; ++t) {
    wait_tiles(n_loaded - 1 - t);   // this wave's loads of tile t have landed
    // Everyone's have, and everyone is done with tile t - 1 (its LDS reads were
    // waited for).  A bare barrier: __syncthreads() would also wait for the
    // loads of the tiles still in flight.
    __builtin_amdgcn_s_barrier();
    if (n_loaded < n_tiles) {       // refill the buffer of tile t - 1
      gload(ld, smem + (n_loaded % kStages) * kTileBytes);
      if (++n_loaded < n_tiles) ld = advance(ld);
    }
    const char* tl = smem + (t % kStages) * kTileBytes;
    const int key0 = kb + cur.lc * kBN;
    const int kend = cur.len;
    if (active) {
    // S^T halves: keys 16 hh + 4 (l/16) + r, head l % 16
    f32x4_t sc[2] = {f32x4_t{0, 0, 0, 0}, f32x4_t{0, 0, 0, 0}};
    // chunk 4 kk + kq of row krow = 16 hh + l % 16: slot 8 (kk / 2) +
    // ((4 (kk % 2) + kq) ^ (krow % 8)), i.e. two per-lane bases plus a constant
    // offset per kk (rows krow and krow + 16 share krow % 8).  The two halves
    // are independent accumulation chains; reads run one k-step ahead.
    {
      const int krow = lane & 15;
      const char* kb0 = tl + krow * kRowBytes + 16 * (kq ^ (krow & 7));
      const char* kb1 = tl + krow * kRowBytes + 16 * ((4 + kq) ^ (krow & 7));
      u32x4_t kr[2][2];
      auto issue = [&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        const char* base = kk & 1 ? kb1 : kb0;
        kr[kk & 1][0] = lds_read16_issue<128 * (kk >> 1)>(base);
        kr[kk & 1][1] = lds_read16_issue<128 * (kk >> 1) + 16 * kRowBytes>(base);
      };
      issue(std::integral_constant<int, 0>{});
      static_for<18>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        if constexpr (kk + 1 < 18) {
          issue(std::integral_constant<int, kk + 1>{});
          lds_wait<2>(kr[kk & 1][0], kr[kk & 1][1]);
        } else {
          lds_wait<0>(kr[kk & 1][0], kr[kk & 1][1]);
        }
        sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[kk & 1][0]), as_bf16x8(qf[kk]), sc[0], 0, 0, 0);
        sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[kk & 1][1]), as_bf16x8(qf[kk]), sc[1], 0, 0, 0);
      });
    }
    const bool tail = key0 + kBN > kend;
    float tmax = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sc[hh][i] * scale2;
        if (tail && key0 + 16 * hh + 4 * kq + i >= kend) v = -INFINITY;
        sc[hh][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = head_max(tmax);
    // lazy rescale: the reference max only moves when a head's max grows by
    // more than kSlack (log2 units); p <= 2^kSlack in between
    if (__any(tmax > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) acc[dt] *= alpha;
    }
    float p[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(sc[0][i] - m_run);
      p[4 + i] = fast_exp2(sc[1][i] - m_run);
      psum += p[i] + p[4 + i];
    }
    l_run += psum;
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
    // V^T fragments in groups of two d-tiles (four reads), one group ahead;
    // dt = 2 g + e reads rows vrow (+16) at slot offset 128 (dt / 4) of vb[dt % 4]
    u32x2_t vr[2][4];
    auto issue = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      constexpr int d0 = 2 * g, d1 = 2 * g + 1;
      vr[g & 1][0] = lds_read_tr_issue<128 * (d0 >> 2)>(vb[d0 & 3]);
      vr[g & 1][1] = lds_read_tr_issue<128 * (d0 >> 2) + 16 * kRowBytes>(vb[d0 & 3]);
      vr[g & 1][2] = lds_read_tr_issue<128 * (d1 >> 2)>(vb[d1 & 3]);
      vr[g & 1][3] = lds_read_tr_issue<128 * (d1 >> 2) + 16 * kRowBytes>(vb[d1 & 3]);
    };
    issue(std::integral_constant<int, 0>{});
    static_for<16>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 1 < 16) {
        issue(std::integral_constant<int, g + 1>{});
        lds_wait<4>(vr[g & 1][0], vr[g & 1][1], vr[g & 1][2], vr[g & 1][3]);
      } else {
        lds_wait<0>(vr[g & 1][0], vr[g & 1][1], vr[g & 1][2], vr[g & 1][3]);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int dt = 2 * g + e;
        const u32x2_t v1 = vr[g & 1][2 * e], v2 = vr[g & 1][2 * e + 1];
        const u32x4_t vf = u32x4_t{v1.x, v1.y, v2.x, v2.y};
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), as_bf16x8(pf), acc[dt], 0, 0, 0);
      }
    });
    }  // active

    if constexpr (kBalanced) {
      // end of this request's keys in the range: emit its segment, start the next
      if ((cur.lc + 1) * kBN >= cur.len && t + 1 < n_tiles) {
        finish(cur);
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0, 0, 0, 0};
        m_run = kNoMax;
        l_run = 0.0f;
        load_q(advance(cur).r);
        gwait();   // q (and every tile load so far) has landed
      }
    }
    if (t + 1 < n_tiles) cur = advance(cur);
  }
  finish(cur);
}

}  // namespace

hipError_t launch_mla_decode(const MlaDecode& a, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  if (a.rank != kRank || a.rope != kRope || a.num_heads % 16 || a.num_heads > 16 * kMaxWaves)
    return hipErrorNotSupported;
  if (a.num_ranges > 0) {
    hipLaunchKernelGGL(mla_kernel<true>, dim3(unsigned(a.num_ranges)), dim3(64 * kMaxWaves), 0, s, a);
    return hipGetLastError();
  }
  const int64_t wgs = int64_t(a.num_seqs) * a.num_splits;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_kernel<false>, dim3(unsigned(wgs)), dim3(64 * kMaxWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
