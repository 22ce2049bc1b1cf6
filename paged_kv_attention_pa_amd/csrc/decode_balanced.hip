// Token-balanced GQA decode over the paged KV cache, bf16, head_dim 128.
//
// Split-KV decode ("第 1 章 注意力后端", §3.1) cuts every request into
// fixed-length splits; with a batch of mixed lengths the number of splits
// rarely divides evenly over the chip, and the last wave of work-groups runs
// a nearly empty machine.  Here the 32-token chunks of all requests form one
// list cut into equal ranges (balanced.hpp); a range finishes the requests
// that lie wholly inside it and leaves an LSE partial for the others, which
// the merge kernel combines.
//
// Work-group: one wave per KV head (up to 8) of one range; the waves walk the
// same chunks.  Loads are contiguous: each instruction fetches a whole 1 KiB
// piece of the work-group's slice of token rows (all its heads), and the
// pieces go through LDS to per-head tiles (a measured 10% more HBM bandwidth
// than each wave gathering its own 256-byte head rows).  Per wave: Q^T stays
// in registers as the B operand of S^T = K Q^T (mfma 16x16x32 bf16, 16 keys
// x 16 query-head columns, G of them used); the P^T registers feed O^T =
// V^T P^T directly.  The registers of chunk c+1 are refilled as soon as
// chunk c's pieces are in LDS, so one chunk of loads is in flight while the
// previous one is computed; two barriers per chunk guard the shared tiles
// (bf16), or one barrier and two sets of tiles (FP8, whose tiles are half
// the size).
#include <type_traits>

#include "balanced.hpp"
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kChunk = kChunkTokens;    // tokens per chunk (one MFMA k-extent)
constexpr int kRow = kD * 2 + 16;       // LDS row of a token: 256 B + 16 B pad
constexpr int kTile = kChunk * kRow;    // per-wave tile (K, then V)
// FP8 tiles hold the codes themselves: 128 B + 16 B pad per token row, and
// the last 16 rows start 16 B further on, so that the transposed reads of
// rows r and r + 16 (one MFMA operand) fall on different LDS banks.  Tiles
// are 128 B past a multiple of 256 B apart: the 16-byte stores of one row of
// two neighbouring heads then use disjoint banks.
constexpr int kRow8 = kD + 16;
constexpr int kTile8 = kChunk * kRow8 + 128;
constexpr int kHeads = 8;               // KV heads (waves) per work-group

// kFp8: the cache holds E4M3 codes (one byte per element).  The loads fetch
// half the bytes and the codes go to LDS as they are (half the LDS traffic
// of widened tiles); each MFMA operand is widened to
// bf16 (exact) as it is read back: 8 codes of a K row (ds_read_b64), or 8
// keys of one V column (ds_read_b64_tr_b8).  The scales fold into the score
// scale (k_scale) and the final normalisation (v_scale), so the products and
// the softmax are the bf16 kernel's.
template <int G, bool kFp8>
__global__ __launch_bounds__(64 * kHeads, 1) void decode_balanced_kernel(DecodeBalanced a) {
  static_assert(G >= 1 && G <= 16, "group must fit the 16 MFMA columns");
  constexpr int kTT = kFp8 ? kTile8 : kTile;   // bytes of one head's K (or V) tile
  // FP8: two sets of tiles, chunk c in set (c - c0) mod 2, so one barrier per
  // chunk suffices (a wave stores chunk c + 1 only after every wave has
  // passed chunk c's barrier, i.e. has finished reading chunk c - 1)
  constexpr int kSets = kFp8 ? 2 : 1;
  constexpr int kSet = 2 * kHeads * kTT;       // K tiles of every head, then V tiles
  __shared__ __align__(16) char smem[kSets * kSet];
  __shared__ int s_wave_sum[kHeads];
  __shared__ int s_start[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int B = a.num_seqs;
  const int cap = a.len_cap;
  const int Hkv = a.num_kv_heads;
  const int n_hg = (Hkv + kHeads - 1) / kHeads;
  const int hg = blockIdx.x % n_hg;
  const int j = blockIdx.x / n_hg;

  const int h = hg * kHeads + wave;   // < Hkv: the launch gives every head group whole waves

  // The step's new tokens, when the decode writes them itself (bf16 cache):
  // the range that holds a request's last chunk writes its row (each wave its
  // KV head: lanes 0-15 the K row, 16-31 the V row) before any load, range 0
  // also those of requests with no keys (no range holds them); after the
  // stores have completed and a barrier, every load of the range sees them
  // (no other range reads a request's last token).
  const bool write_new = !kFp8 && a.k_new != nullptr;
  const int64_t new_tok_bytes = int64_t(a.num_kv_heads) * kD * 2;
  auto write_token = [&](int r) {
    const int64_t slot = uniform_load(a.slots + r);
    if (slot < 0 || slot >= a.num_blocks * a.block_size || lane >= 32) return;
    const int plane = lane >> 4, c = lane & 15;
    const int64_t blk = slot / a.block_size, off = slot - blk * a.block_size;
    const char* src = static_cast<const char*>(plane ? a.v_new : a.k_new) +
                      (int64_t(r) * a.num_kv_heads + h) * (kD * 2) + 16 * c;
    char* dst = static_cast<char*>(const_cast<void*>(a.cache)) +
                ((blk * 2 + plane) * a.block_size + off) * new_tok_bytes + h * (kD * 2) + 16 * c;
    *reinterpret_cast<u32x4_t*>(dst) = load16(src);
  };
  if (write_new && j == 0) {
    for (int r = 0; r < B; ++r)
      if (clamp_len(uniform_load(a.seq_lens + r), cap) == 0) write_token(r);
  }

  int c0, c1, n_chunks;   // no overhead units: chunks c0 .. c1 - 1
  ChunkPos cur;
  if (!balanced_range(a.seq_lens, B, cap, a.num_ranges, j, j == 0 && hg == 0, a.cu, s_wave_sum,
                      s_start, c0, c1, n_chunks, cur))
    return;
  if (write_new) {
    ChunkPos p = cur;   // holds chunk c0
    for (;;) {
      const int n = chunks_of(p.len);
      const int last = p.base + n - 1;   // the request's last chunk
      if (last >= c1) break;             // held by a later range
      write_token(p.r);
      if (last + 1 >= c1) break;
      p = next_chunk(ChunkPos{p.r, n - 1, p.len, p.base}, a.seq_lens, cap, B);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the stores have completed
    __syncthreads();
  }

  const int li = lane & 15;   // MFMA row/column index; 16-byte chunk of a loaded row
  const int kq = lane >> 4;   // 16-lane group; token within a 4-token load
  const int Hq = a.num_q_heads;
  const int bs = a.block_size;
  const int64_t tok_stride = int64_t(Hkv) * kD;
  const int64_t kv_stride = int64_t(bs) * tok_stride;
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  const float scale2 = (kFp8 ? a.scale * a.k_scale : a.scale) * kLog2e;
  constexpr int kElem = kFp8 ? 1 : 2;           // cache bytes per element
  constexpr int kLoads = kFp8 ? 4 : 8;          // 16-byte loads per lane per plane and chunk
  constexpr int kRowShift = kFp8 ? 7 : 8;       // log2 of a head row's cache bytes

  const int waves = blockDim.x >> 6;
  const char* const a_base = smem + wave * kTile + li * kRow + 16 * kq;             // K: row 16 sub + li
  const char* const tr_base = smem + (kHeads + wave) * kTile + (4 * kq + (li >> 2)) * kRow + 8 * (li & 3);
  // FP8 tiles.  K operand of S^T: row 16 sub + li, codes 32 kk + 8 kq .. +7.
  // V^T operand: ds_read_b64_tr_b8 hands lane li of a 16-lane group byte li
  // of each of 8 rows, row k being the 8-byte chunks of lanes 2k and 2k + 1;
  // lane pair k points at key 4 kq + (k mod 4) + 16 (k / 4), dims 16 dt ..
  // 16 dt + 15, so lane li gets dim 16 dt + li of the keys in P^T's order
  // (4 kq + i, then 16 + 4 kq + i).
  const char* const k8_base = smem + wave * kTile8 + li * kRow8 + 8 * kq;
  const int vk = 4 * kq + ((li >> 1) & 3) + 16 * (li >> 3);
  const char* const v8_base = smem + (kHeads + wave) * kTile8 + vk * kRow8 + 16 * (vk >> 4) + 8 * (li & 1);
  // Loads are contiguous 1 KiB pieces of the work-group's slice of a token
  // row (waves x 256 B): instruction i of wave w is piece I = w + waves i,
  // lane l its bytes 16 l .. 16 l + 15.  Piece I covers tokens (1024 I) /
  // slice .., byte (1024 I + 16 l) % slice of the slice, i.e. head
  // byte / 256, 16-byte chunk (byte % 256) / 16.
  const int lw = waves == 8 ? 3 : waves == 4 ? 2 : waves == 2 ? 1 : 0;
  const int sh = kRowShift + lw;               // log2 of the slice bytes
  const char* cache_b = static_cast<const char*>(a.cache) + int64_t(hg) * kHeads * kD * kElem;
  const int64_t tok_bytes = tok_stride * kElem, kv_bytes = kv_stride * kElem;

  // Q^T columns: lane li holds query head h G + (li mod G); the columns past G
  // repeat real rows and their results are never stored.
  auto load_q = [&](int r, u32x4_t (&qf)[4]) {
    const uint16_t* qp = qbase + (int64_t(r) * Hq + int64_t(h) * G + (li & (G - 1))) * kD + 8 * kq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = load16(qp + 32 * kk);
  };
  // Pieces of chunk p.  Tokens past the request's end re-read its last
  // token (finite data, masked below); the loads are unconditional so the
  // waits stay exact.
  // The scalar address math stays small (the scalar unit is shared by the
  // compute unit's four SIMDs): page of a token by a shift when the block
  // size is a power of two, byte offsets within a page in 32 bits.
  const bool bs_pow2 = (bs & (bs - 1)) == 0;
  const int bs_shift = __builtin_ctz(unsigned(bs));
  const uint64_t page_bytes = 2 * uint64_t(bs) * uint64_t(tok_bytes);
  const uint32_t tok32 = uint32_t(tok_bytes);
  const uint32_t nblk = uint32_t(min(a.num_blocks, int64_t(INT32_MAX)));
  // K and V pieces of chunk p: one address per piece for both planes (the V
  // piece is kv_bytes on), so the page lookups and the scalar address math
  // are done once.
  // A load past the range's last chunk (dummy) keeps the wait counts exact
  // but reads the first token row of block 0, the same bytes for every
  // work-group, which stay in L2 instead of costing HBM bytes.
  auto load_kv = [&](const ChunkPos& p, bool dummy, u32x4_t (&kdst)[kLoads],
                     u32x4_t (&vdst)[kLoads]) {
    const int32_t* table = a.block_table + int64_t(p.r) * a.max_blocks;
    const int len = max(p.len, 1);   // positions always hold keys; keeps every index >= 0
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int I = wave + waves * i;
      const int lin = I * 1024 + 16 * lane;
      const int tl_first = (I * 1024) >> sh;                       // first token of the piece
      const int tok_first = min(p.lc * kChunk + tl_first, len - 1);
      const int page = bs_pow2 ? tok_first >> bs_shift : tok_first / bs;
      uint32_t blk = uint32_t(uniform_load(table + page));
      blk = blk < nblk ? blk : 0u;   // negative ids wrap high
      const int tok = min(p.lc * kChunk + (lin >> sh), len - 1);
      const int byte = lin & ((1 << sh) - 1);
      // non-temporal: every cache byte is read once, so it need not displace
      // anything in L2 or the MALL (81% against 72% of HBM peak on the
      // headline batch)
      blk = dummy ? 0u : blk;
      const uint32_t off = (dummy ? 0u : uint32_t(tok - page * bs) * tok32) + uint32_t(byte);
      // page bases are scalars; the lane offset is one 32-bit register
      const char* kpage = cache_b + blk * page_bytes;
      const char* vpage = kpage + kv_bytes;
      kdst[i] = load16_stream(kpage + off);
      vdst[i] = load16_stream(vpage + off);
    }
  };
  // LDS position of this lane's piece i (head tile, token row, byte of the
  // bf16 row)
  auto lds_off = [&](int i) {
    const int lin = (wave + waves * i) * 1024 + 16 * lane;
    const int byte = lin & ((1 << sh) - 1);
    const int t = lin >> sh;
    if constexpr (kFp8)
      return (byte >> kRowShift) * kTile8 + t * kRow8 + 16 * (t >> 4) + (byte & ((1 << kRowShift) - 1));
    else
      return (byte >> kRowShift) * kTile + t * kRow + (byte & ((1 << kRowShift) - 1));
  };

  ChunkPos nxt = c0 + 1 < c1 ? next_chunk(cur, a.seq_lens, cap, B) : cur;

  u32x4_t qf[4];
  load_q(cur.r, qf);
  u32x4_t kr[kLoads], vr[kLoads];
  load_kv(cur, false, kr, vr);

  f32x4_t acc[8];   // O^T: d = 16 dt + 4 kq + i, head column li
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0, 0, 0, 0};
  float m_run = kNoMax, l_run = 0.0f;

  // One chunk; set (a compile-time constant) names its tiles.
  auto step = [&](const int c, auto set) {
    constexpr int ST = decltype(set)::value * kSet;
    // this chunk's pieces into every head's K and V tiles; once all waves'
    // are there, the registers are refilled with the next chunk
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int o = ST + lds_off(i);
      *reinterpret_cast<u32x4_t*>(smem + o) = kr[i];
      *reinterpret_cast<u32x4_t*>(smem + kHeads * kTT + o) = vr[i];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS stores are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    load_kv(nxt, c + 1 >= c1, kr, vr);
    f32x4_t sc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sc[sub] = f32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4_t kf;
        if constexpr (kFp8) {
          const u32x2_t c8 = *reinterpret_cast<const u32x2_t*>(k8_base + ST + sub * (16 * kRow8 + 16) + 32 * kk);
          kf = u32x4_t{fp8x2_to_bf16x2<false>(c8[0]), fp8x2_to_bf16x2<true>(c8[0]),
                       fp8x2_to_bf16x2<false>(c8[1]), fp8x2_to_bf16x2<true>(c8[1])};
        } else {
          kf = *reinterpret_cast<const u32x4_t*>(a_base + 16 * sub * kRow + 64 * kk);
        }
        sc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[kk]), sc[sub], 0, 0, 0);
      }
    }
    const bool new_request = nxt.lc == 0 && c + 1 < c1;
    if (new_request) load_q(nxt.r, qf);

    // online softmax over this chunk (base 2); keys past the request end masked
    const int tok0 = cur.lc * kChunk;
    const bool tail = tok0 + kChunk > cur.len;
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sc[sub][i] * scale2;
        if (tail && tok0 + 16 * sub + 4 * kq + i >= cur.len) v = -INFINITY;
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
    // O^T += V^T P^T: lane li of group kq reads 4 bf16 of token row
    // 4 kq + li / 4 (and +16) at dims 16 dt + 4 (li % 4).
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      u32x4_t vf;
      if constexpr (kFp8) {
        const u32x2_t c8 = lds_read_tr8(v8_base + ST + 16 * dt);
        vf = u32x4_t{fp8x2_to_bf16x2<false>(c8[0]), fp8x2_to_bf16x2<true>(c8[0]),
                     fp8x2_to_bf16x2<false>(c8[1]), fp8x2_to_bf16x2<true>(c8[1])};
      } else {
        const uint2 v1 = lds_read_tr(tr_base + 32 * dt);
        const uint2 v2 = lds_read_tr(tr_base + 16 * kRow + 32 * dt);
        vf = u32x4_t{v1.x, v1.y, v2.x, v2.y};
      }
      acc[dt] *= alpha;
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), as_bf16x8(pf), acc[dt], 0, 0, 0);
    }

    // end of this request's keys within the range: emit its segment
    if (tok0 + kChunk >= cur.len || c + 1 == c1) {
      const float l_w = l_run + lane_xor(l_run, 16);
      const float l_tot = l_w + lane_xor(l_w, 32);
      const float inv = (kFp8 ? a.v_scale : 1.0f) / l_tot;
      const float lse_nat = (m_run + fast_log2(l_tot)) * kLn2;
      const bool whole = cur.base >= c0 && cur.base + chunks_of(cur.len) <= c1;
      if (li < G) {
        const int64_t hrow = int64_t(h) * G + li;
        if (whole) {
          const int64_t row = int64_t(cur.r) * Hq + hrow;
          uint16_t* op = static_cast<uint16_t*>(a.out) + row * kD + 4 * kq;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            uint2 w;
            w.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
            w.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
            *reinterpret_cast<uint2*>(op + 16 * dt) = w;
          }
          if (kq == 0 && a.lse) a.lse[row] = lse_nat;
        } else {
          float* pp = a.part + (int64_t(j + cur.r) * Hq + hrow) * (kD + 4);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            *reinterpret_cast<f32x4_t*>(pp + 16 * dt + 4 * kq) = acc[dt] * inv;
          if (kq == 0) pp[kD] = lse_nat;
        }
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0, 0, 0, 0};
      m_run = kNoMax;
      l_run = 0.0f;
    }
    cur = nxt;
    if (c + 2 < c1) nxt = next_chunk(nxt, a.seq_lens, cap, B);
    if constexpr (kSets == 1) __builtin_amdgcn_s_barrier();   // every wave is done reading the tiles
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, kSets - 1>;
  if constexpr (kSets == 1) {
    for (int c = c0; c < c1; ++c) step(c, Set0{});
  } else {
    const int pairs = (c1 - c0) >> 1;
    int c = c0;
    for (int t = 0; t < pairs; ++t, c += 2) {
      step(c, Set0{});
      step(c + 1, Set1{});
    }
    if (c < c1) step(c, Set0{});
  }
}

// Combine the segments of requests that cross ranges.  One work-group per
// (request, query head): DV / 4 threads (4 dims each) cover a row; the
// 1024 / DV groups of them take every k-th segment and keep a running
// (max, sum, output) each, merged through LDS at the end.
template <int DV>
__global__ __launch_bounds__(256) void balanced_merge_kernel(BalancedMerge a) {
  constexpr int kGroupThreads = DV / 4;
  constexpr int kGroups = 256 / kGroupThreads;
  constexpr int kRowF = DV + 4;               // fp32 per segment row, lse at DV
  __shared__ float s_m[kGroups], s_l[kGroups];
  __shared__ __align__(16) float s_o[kGroups][DV];
  const int Hq = a.num_q_heads;
  const int r = blockIdx.x / Hq;
  const int hq = blockIdx.x % Hq;
  const int g = threadIdx.x / kGroupThreads;
  const int d = 4 * (threadIdx.x % kGroupThreads);
  const int B = a.num_seqs;
  const int total = a.cu[B];
  const int cb = a.cu[r];
  const int ce = a.cu[r + 1];
  const int64_t row = int64_t(r) * Hq + hq;
  uint2* op = reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * DV + d);
  if (cb == ce) {   // no keys: out 0, lse -inf
    if (g == 0) *op = uint2{0u, 0u};
    if (a.lse && threadIdx.x == 0) a.lse[row] = -INFINITY;
    return;
  }
  const int nr = min(a.num_ranges, total);
  constexpr int kW = DV == 128 ? 0 : kMlaRangeOverhead;   // GQA or MLA (rank 256) ranges
  const int j0 = range_of_unit(cb + kW, nr, total);
  const int j1 = range_of_unit(ce - 1, nr, total);
  if (j0 == j1) return;   // written by its range
  const int64_t step = int64_t(Hq) * kRowF;
  const float* p0 = a.part + (int64_t(j0 + r) * Hq + hq) * kRowF;
  float m = -INFINITY, l = 0.0f;
  f32x4_t o = f32x4_t{0, 0, 0, 0};
#pragma unroll 4
  for (int jj = g; jj <= j1 - j0; jj += kGroups) {
    const float* pp = p0 + jj * step;
    const float lj = pp[DV];
    const f32x4_t oj = *reinterpret_cast<const f32x4_t*>(pp + d);
    const float mn = fmaxf(m, lj);
    const float c = fast_exp2((m - mn) * kLog2e);   // 0 while m = -inf
    const float w = fast_exp2((lj - mn) * kLog2e);
    l = fmaf(l, c, w);
    o = o * c + w * oj;
    m = mn;
  }
  if (threadIdx.x % kGroupThreads == 0) {
    s_m[g] = m;
    s_l[g] = l;
  }
  *reinterpret_cast<f32x4_t*>(&s_o[g][d]) = o;
  __syncthreads();
  if (g != 0) return;
  float mm = s_m[0];
#pragma unroll
  for (int k = 1; k < kGroups; ++k) mm = fmaxf(mm, s_m[k]);
  float den = 0.0f;
  f32x4_t acc = f32x4_t{0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < kGroups; ++k) {
    const float w = fast_exp2((s_m[k] - mm) * kLog2e);   // 0 for a group without segments
    den = fmaf(s_l[k], w, den);
    acc += w * *reinterpret_cast<const f32x4_t*>(&s_o[k][d]);
  }
  const float inv = 1.0f / den;
  *op = uint2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (a.lse && threadIdx.x == 0) a.lse[row] = mm + fast_log2(den) * kLn2;
}

// The 512-wide (MLA) merge: requests cross few ranges but rows are long.
// One work-group per (request, 8 heads): 32 threads per head, 16 dims each,
// one running (max, sum, output) per thread over the request's segments.
__global__ __launch_bounds__(256) void balanced_merge512_kernel(BalancedMerge a) {
  constexpr int DV = 512, kRowF = DV + 4, kHeadsPerGroup = 8;
  const int Hq = a.num_q_heads;
  const int nhb = (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int r = blockIdx.x / nhb;
  const int hq = (blockIdx.x % nhb) * kHeadsPerGroup + (threadIdx.x >> 5);
  if (hq >= Hq) return;
  const int d = 16 * (threadIdx.x & 31);
  const int B = a.num_seqs;
  const int total = a.cu[B];
  const int cb = a.cu[r];
  const int ce = a.cu[r + 1];
  const int64_t row = int64_t(r) * Hq + hq;
  u32x4_t* op = reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.out) + row * DV + d);
  if (cb == ce) {   // no keys: out 0, lse -inf
    op[0] = u32x4_t{0, 0, 0, 0};
    op[1] = u32x4_t{0, 0, 0, 0};
    if (a.lse && (threadIdx.x & 31) == 0) a.lse[row] = -INFINITY;
    return;
  }
  const int nr = min(a.num_ranges, total);
  const int j0 = range_of_unit(cb + kMlaRangeOverhead, nr, total);   // MLA ranges
  const int j1 = range_of_unit(ce - 1, nr, total);
  if (j0 == j1) return;   // written by its range
  const int64_t step = int64_t(Hq) * kRowF;
  const float* p0 = a.part + (int64_t(j0 + r) * Hq + hq) * kRowF;
  float m = -INFINITY, l = 0.0f;
  f32x4_t o[4] = {f32x4_t{0, 0, 0, 0}, f32x4_t{0, 0, 0, 0}, f32x4_t{0, 0, 0, 0}, f32x4_t{0, 0, 0, 0}};
#pragma unroll 2
  for (int jj = 0; jj <= j1 - j0; ++jj) {
    const float* pp = p0 + jj * step;
    const float lj = pp[DV];
    f32x4_t oj[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) oj[k] = *reinterpret_cast<const f32x4_t*>(pp + d + 4 * k);
    const float mn = fmaxf(m, lj);
    const float c = fast_exp2((m - mn) * kLog2e);   // 0 while m = -inf
    const float w = fast_exp2((lj - mn) * kLog2e);
    l = fmaf(l, c, w);
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = o[k] * c + w * oj[k];
    m = mn;
  }
  const float inv = 1.0f / l;
  op[0] = u32x4_t{pack_bf16x2(o[0][0] * inv, o[0][1] * inv), pack_bf16x2(o[0][2] * inv, o[0][3] * inv),
                  pack_bf16x2(o[1][0] * inv, o[1][1] * inv), pack_bf16x2(o[1][2] * inv, o[1][3] * inv)};
  op[1] = u32x4_t{pack_bf16x2(o[2][0] * inv, o[2][1] * inv), pack_bf16x2(o[2][2] * inv, o[2][3] * inv),
                  pack_bf16x2(o[3][0] * inv, o[3][1] * inv), pack_bf16x2(o[3][2] * inv, o[3][3] * inv)};
  if (a.lse && (threadIdx.x & 31) == 0) a.lse[row] = m + fast_log2(l) * kLn2;
}

}  // namespace

int balanced_num_ranges(int num_kv_heads, int num_cus) {
  if (num_kv_heads < 1) num_kv_heads = 1;
  if (num_cus < 1) num_cus = 1;
  const int waves = num_kv_heads < kHeads ? num_kv_heads : kHeads;
  const int n_hg = (num_kv_heads + kHeads - 1) / kHeads;
  const int64_t nr = int64_t(num_cus) * kHeads / (int64_t(waves) * n_hg);   // 8 waves per CU
  return int(nr < 1 ? 1 : nr);
}

size_t balanced_cu_bytes(int num_seqs) { return (size_t(num_seqs + 1) * 4 + 255) / 256 * 256; }

hipError_t launch_decode_balanced(const DecodeBalanced& a, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int n_hg = (a.num_kv_heads + kHeads - 1) / kHeads;
  const int waves = a.num_kv_heads < kHeads ? a.num_kv_heads : kHeads;
  const dim3 grid{unsigned(int64_t(a.num_ranges) * n_hg)}, block{unsigned(64 * waves)};
  if (a.fp8) {
    switch (G) {
      case 1: hipLaunchKernelGGL((decode_balanced_kernel<1, true>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((decode_balanced_kernel<2, true>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((decode_balanced_kernel<4, true>), grid, block, 0, s, a); break;
      case 8: hipLaunchKernelGGL((decode_balanced_kernel<8, true>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_balanced_kernel<1, false>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_balanced_kernel<2, false>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_balanced_kernel<4, false>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_balanced_kernel<8, false>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_balanced_merge(const BalancedMerge& a, hipStream_t s) {
  if (a.head_dim == 128) {
    const dim3 grid{unsigned(int64_t(a.num_seqs) * a.num_q_heads)}, block{256};
    hipLaunchKernelGGL((balanced_merge_kernel<128>), grid, block, 0, s, a);
  } else if (a.head_dim == 256) {
    const dim3 grid{unsigned(int64_t(a.num_seqs) * a.num_q_heads)}, block{256};
    hipLaunchKernelGGL((balanced_merge_kernel<256>), grid, block, 0, s, a);
  } else if (a.head_dim == 512) {
    const dim3 grid{unsigned(int64_t(a.num_seqs) * ((a.num_q_heads + 7) / 8))}, block{256};
    hipLaunchKernelGGL(balanced_merge512_kernel, grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
