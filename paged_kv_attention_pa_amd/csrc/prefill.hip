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
// element.  Work-group ids keep each (request, KV head) on one XCD (L2 reuse
// of its K/V), longest q tile first.
#include <type_traits>

#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kBM = 128;           // query rows per work-group
constexpr int kBN = 64;            // keys per tile
constexpr int kRowBytes = kD * 2;        // 256 B per key row (unpadded, swizzled)
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KiB
constexpr int kTileLoads = kBN * kRowBytes / 1024;  // 16 wave-wide 16-byte loads per tile
constexpr int kXcds = 8;           // accelerator dies work-groups are dealt to
constexpr float kSlack = 8.0f;     // lazy-rescale headroom, log2 units
constexpr int kPrefillLead = 2;    // ping-pong prefill: periods between a gather and its use
// 16-byte chunk c of key row r sits in slot c ^ swz(r) of the row, with
// swz(r) = 4 (r % 4) + (r / 4) % 4 (a permutation of r % 16).  Rows are
// 256 B, so every row starts on the same bank, and the 64 banks are the 16
// slots of a row.  A 16-lane phase of a K-fragment read (16 rows, one
// chunk) then hits 16 distinct slots; a 32-lane phase of a V^T transpose
// read (4 consecutive rows, 4 consecutive chunks) puts each row in its own
// 4-slot group.  Both are conflict-free.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// kPrefix = false: varlen prefill, one (request, query head, 128-row q tile)
// per work-group, out / lse written directly.
// kPrefix = true: the shared prefix of a cascade -- the batch's query rows,
// each (token, head of the group) pair a row (row = token * G + head), against
// one key range of the prefix, fp32 partials out.
// kFp8 (varlen prefill only): the cache holds E4M3 codes.  Each thread loads
// its 16-byte pieces of tile t + 1 into registers while tile t is computed,
// and after a barrier widens them to bf16 (exact) into the single tile
// buffer; k_scale folds into the score scale and v_scale into the final
// normalisation.
template <bool kPrefix, bool kFp8>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillVarlen a) {
  static_assert(!(kPrefix && kFp8), "the shared-prefix pass reads a bf16 cache");
  __shared__ __align__(16) char smem[4 * kTileBytes];   // 2 x (K tile, V tile)
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int tid = threadIdx.x;
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int bs = a.block_size;
  const int id = blockIdx.x;
  const int xcd = id % kXcds;
  const int slot = id / kXcds;

  int r, h, q_start, L, q0, C, kvh, kv_end, t_begin = 0, split = 0;
  if constexpr (!kPrefix) {
    // work-group -> (request, KV head, q tile, head of the group).  Work-groups
    // are dealt to the 8 XCDs round-robin by id, so ids are arranged such that
    // every q tile and query head of one (request, KV head) pair land on the
    // same XCD, one after another: that pair's K/V (at most a few MB) is read
    // from HBM once and then served by that XCD's L2.  Within a pair, the
    // longest (last) q tiles go first.
    const int n_qt = (a.max_query_len + kBM - 1) / kBM;
    const int per_pair = n_qt * G;
    const int pair = (slot / per_pair) * kXcds + xcd;          // (request, KV head)
    if (pair >= a.num_seqs * a.num_kv_heads) return;
    const int local = slot % per_pair;
    r = pair / a.num_kv_heads;
    kvh = pair % a.num_kv_heads;
    const int qt = n_qt - 1 - local / G;
    h = kvh * G + local % G;
    q_start = min(max(a.query_start_loc[r], 0), a.num_tokens);
    L = min(min(a.query_start_loc[r + 1] - q_start, a.max_query_len), a.num_tokens - q_start);
    const int S = min(a.seq_lens[r], a.max_blocks * bs);
    q0 = qt * kBM;
    if (q0 >= L || L <= 0) return;
    C = S - L;                    // keys before the chunk
    // keys this work-group may see
    kv_end = S;
    if (a.causal) kv_end = min(S, max(0, C + min(q0 + kBM, L)));
  } else {
    // work-group -> (KV head, key range, row tile): the row tiles of one
    // (KV head, key range) pair share that range's K/V and sit on one XCD.
    const int n_qt = (a.num_tokens * G + kBM - 1) / kBM;
    const int pair = (slot / n_qt) * kXcds + xcd;              // (KV head, key range)
    if (pair >= a.num_kv_heads * a.prefix_splits) return;
    kvh = pair / a.prefix_splits;
    split = pair % a.prefix_splits;
    r = 0;                        // the prefix's pages: row 0 of the table
    h = kvh * G;                  // per-lane head set below
    q_start = 0;
    L = a.num_tokens * G;         // rows
    q0 = (slot % n_qt) * kBM;
    C = 0;
    const int key_begin = split * a.split_keys;
    kv_end = min(min(a.prefix_len, a.max_blocks * bs), key_begin + a.split_keys);
    if (key_begin >= kv_end) return;
    t_begin = key_begin / kBN;
  }
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // ---- Q fragments (B operand of S^T): row = l % 32, d chunk = 16 kk + 8 (l / 32)
  const int my_row = q0 + wave * 32 + (lane & 31);
  const bool row_ok = my_row < L;
  int64_t q_off;   // element offset of this lane's query row
  if constexpr (!kPrefix) {
    q_off = (int64_t(q_start) + (row_ok ? my_row : 0)) * Hq * kD + int64_t(h) * kD;
  } else {
    const int row = row_ok ? my_row : 0;
    const int tok = row / G;       // G is a power of two
    h = kvh * G + (row - tok * G);
    q_off = (int64_t(tok) * Hq + h) * kD;
  }
  u32x4_t qf[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + q_off + 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = row_ok ? load16(qp + 16 * kk) : u32x4_t{0, 0, 0, 0};
  }

  // ---- gather of one K/V tile straight into LDS (global_load_lds_dwordx4):
  // 16 wave-wide loads per half, wave w issuing loads w, w + 4, w + 8, w + 12.
  // Load j fills rows 4 j .. 4 j + 3 (lane i: row 4 j + i / 16, slot i % 16,
  // which holds chunk slot ^ swz(row)).  The four rows of a load share one
  // page (16-key groups are 16-aligned, pages are multiples of 16): the page
  // id is a wave-uniform scalar load, the page address a scalar base, and the
  // lane's offset within the group a per-lane constant.  Keys past kv_end
  // re-read key kv_end - 1 (finite, masked out below).
  const int64_t tok_bytes = int64_t(a.num_kv_heads) * kD * 2;
  const int64_t kv_bytes = int64_t(bs) * tok_bytes;
  const char* cache_h = static_cast<const char*>(a.cache) + int64_t(kvh) * kD * 2;
  const int32_t* table = a.block_table + int64_t(r) * a.max_blocks;
  // byte offset of this lane's 16 bytes within its 16-key group, per load jj
  // (the same for every tile except the last group of the keys)
  uint32_t lane_off[kTileLoads / 4];
#pragma unroll
  for (int jj = 0; jj < kTileLoads / 4; ++jj) {
    const int row = 4 * (wave + 4 * jj) + (lane >> 4);
    lane_off[jj] = uint32_t((row & 15) * tok_bytes + 16 * ((lane & 15) ^ swz(row)));
  }
  const int last16 = ((kv_end - 1) / 16) * 16;
  // Scalar address math per load, kept small: the scalar unit is shared by
  // the compute unit's four SIMDs, and a division plus 64-bit products per
  // load would keep it busy for most of a tile.  Page and row of a key come
  // from shifts when the block size is a power of two; byte offsets within a
  // page fit 32 bits (a page is 2 x bs x Hkv x 256 bytes).
  const bool bs_pow2 = (bs & (bs - 1)) == 0;
  const int bs_shift = __builtin_ctz(unsigned(bs));
  const uint32_t tok32 = uint32_t(tok_bytes);
  const uint32_t page_bytes = 2u * uint32_t(bs) * tok32;   // one page: K rows, then V rows
  const uint32_t kv32 = uint32_t(kv_bytes);                // V rows of a page, after its K rows
  const uint32_t nblk = uint32_t(min(a.num_blocks, int64_t(INT32_MAX)));
  auto gload = [&](int tile, char* kdst) {
    char* vdst = kdst + kTileBytes;
    // the four 16-key groups of the tile: page ids first (one wait for all)
    uint32_t blk[4], in_page[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int key16 = min(tile * kBN + 16 * jj, last16);
      const int page = bs_pow2 ? key16 >> bs_shift : key16 / bs;
      in_page[jj] = uint32_t(key16 - page * bs);
      blk[jj] = uint32_t(uniform_load(table + page));
    }
    const bool tail = tile * kBN + kBN > kv_end;   // wave-uniform
#pragma unroll
    for (int jj = 0; jj < kTileLoads / 4; ++jj) {
      const int j = wave + 4 * jj;   // load j: rows 4 j .. 4 j + 3 of group j / 4 = jj (4 waves)
      const uint32_t b = blk[jj] < nblk ? blk[jj] : 0u;   // negative ids wrap high
      const char* base = cache_h + uint64_t(b) * page_bytes;
      uint32_t off = lane_off[jj] + in_page[jj] * tok32;
      if (tail) {   // keys past kv_end re-read key kv_end - 1
        const int key16 = min(tile * kBN + 16 * jj, last16);
        const int row = 4 * j + (lane >> 4);
        off = in_page[jj] * tok32 +
              uint32_t(min(row & 15, kv_end - 1 - key16) * tok_bytes + 16 * ((lane & 15) ^ swz(row)));
      }
      typedef __attribute__((address_space(3))) void* lds_ptr;
      __builtin_amdgcn_global_load_lds(base + off, (lds_ptr)(kdst + 1024 * j), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(base + kv32 + off, (lds_ptr)(vdst + 1024 * j), 16, 0, 0);
    }
  };
  auto gwait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  // ---- FP8: register gather.  Thread piece p = tid + 256 i (i = 0, 1) of a
  // plane is key p / 8, codes 16 (p % 8) .. + 15 of its head row; its key's
  // 16-key group is (p / 8) / 16 = 2 i + tid / 128, whose page id is one of
  // the tile's four scalar loads.
  const int64_t f8_tok = int64_t(a.num_kv_heads) * kD;       // bytes per token (codes)
  const uint32_t f8_tok32 = uint32_t(f8_tok);
  const uint32_t f8_page = 2u * uint32_t(bs) * f8_tok32;
  const uint32_t f8_kv = uint32_t(bs) * f8_tok32;
  const char* f8_cache_h = static_cast<const char*>(a.cache) + int64_t(kvh) * kD;
  u32x4_t f8r[4];   // K pieces i = 0, 1, then V pieces
  auto rload = [&](int tile) {
    uint32_t blk[4], in_page[4];
    int key16[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      key16[jj] = min(tile * kBN + 16 * jj, last16);
      const int page = bs_pow2 ? key16[jj] >> bs_shift : key16[jj] / bs;
      in_page[jj] = uint32_t(key16[jj] - page * bs);
      blk[jj] = uint32_t(uniform_load(table + page));
    }
    const bool tail = tile * kBN + kBN > kv_end;   // wave-uniform
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int key = p >> 3, c8 = p & 7;
      const int grp = 2 * i + (tid >> 7);
      // the lane's group among the two this piece can fall in
      const uint32_t bg = (tid >> 7) ? blk[2 * i + 1] : blk[2 * i];
      const uint32_t ip = (tid >> 7) ? in_page[2 * i + 1] : in_page[2 * i];
      const int k16 = (tid >> 7) ? key16[2 * i + 1] : key16[2 * i];
      (void)grp;
      int rr = key & 15;
      if (tail) rr = min(rr, kv_end - 1 - k16);
      const uint32_t b = bg < nblk ? bg : 0u;
      const char* base = f8_cache_h + uint64_t(b) * f8_page;
      const uint32_t off = (ip + uint32_t(rr)) * f8_tok32 + 16u * uint32_t(c8);
      f8r[i] = load16(base + off);
      f8r[2 + i] = load16(base + f8_kv + off);
    }
  };
  auto rstore = [&](char* kdst) {
    char* vdst = kdst + kTileBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int key = p >> 3, c8 = p & 7;
      const int o0 = key * kRowBytes + 16 * ((2 * c8) ^ swz(key));
      const int o1 = key * kRowBytes + 16 * ((2 * c8 + 1) ^ swz(key));
      u32x4_t lo, hi;
      fp8x16_to_bf16(f8r[i], lo, hi);
      *reinterpret_cast<u32x4_t*>(kdst + o0) = lo;
      *reinterpret_cast<u32x4_t*>(kdst + o1) = hi;
      fp8x16_to_bf16(f8r[2 + i], lo, hi);
      *reinterpret_cast<u32x4_t*>(vdst + o0) = lo;
      *reinterpret_cast<u32x4_t*>(vdst + o1) = hi;
    }
  };

  const float scale2 = (kFp8 ? a.scale * a.k_scale : a.scale) * kLog2e;
  float m_run = kNoMax;   // running max (base-2 domain) of row my_row
  float l_run = 0.0f;     // this lane's share of the running sum
  f32x16_t acc[4];        // O^T tiles: d = 32 dt + 8 (r/4) + 4 (l/32) + r%4
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;

  if constexpr (kFp8) {
    if (n_tiles > t_begin) {
      rload(t_begin);
      rstore(smem);
    }
  } else {
    if (n_tiles > t_begin) {
      gload(t_begin, smem);
      gwait();
    }
  }
  __syncthreads();

  const bool causal = kPrefix ? false : a.causal;
  const int row_abs = C + my_row;         // last key this row may see (causal)
  for (int t = t_begin; t < n_tiles; ++t) {
    const int buf = kFp8 ? 0 : (t - t_begin) & 1;
    if (t + 1 < n_tiles) {   // in flight below
      if constexpr (kFp8) rload(t + 1);
      else gload(t + 1, smem + (buf ^ 1) * 2 * kTileBytes);
    }
    const char* kt = smem + buf * 2 * kTileBytes;
    const char* vt = kt + kTileBytes;
    const int key0 = t * kBN;

    // S^T for two 32-key halves (two independent accumulation chains).  Chunk
    // 2 kk + (l / 32) of row 32 hh + l % 32 sits in slot (2 kk + l / 32) ^
    // swz(l % 32); the second half is a constant 32 rows further.  The LDS
    // reads run two k-steps ahead of the MFMAs.
    f32x16_t s[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[hh][i] = 0.0f;
    {
      constexpr int kQD = 2;   // k-steps of reads in flight ahead of the MFMAs
      const char* krow = kt + (lane & 31) * kRowBytes;
      u32x4_t kr[kQD + 1][2];
      auto issue = [&](auto kc) {
        constexpr int kk = decltype(kc)::value, b = kk % (kQD + 1);
        const char* p = krow + 16 * ((2 * kk + (lane >> 5)) ^ swz(lane & 31));
        kr[b][0] = lds_read16_issue<0>(p);
        kr[b][1] = lds_read16_issue<32 * kRowBytes>(p);
      };
      static_for<kQD>([&](auto kc) { issue(kc); });
      static_for<8>([&](auto kc) {
        constexpr int kk = decltype(kc)::value, b = kk % (kQD + 1);
        if constexpr (kk + kQD < 8) issue(std::integral_constant<int, kk + kQD>{});
        constexpr int kLater = 2 * (kk + kQD < 8 ? kQD : 7 - kk);   // 2 reads per later step
        lds_wait<kLater>(kr[b][0], kr[b][1]);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[b][0]), as_bf16x8(qf[kk]), s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[b][1]), as_bf16x8(qf[kk]), s[1], 0, 0, 0);
      });
    }

    // Online softmax update for this tile.  Diagonal and tail tiles (wave-
    // uniform `need_mask`) take the masked path; interior tiles skip every
    // mask test.  The running max m_run is a reference that only moves when a
    // tile's max exceeds it by more than kSlack (log2 units): until then the
    // accumulator needs no rescale and P stays below 2^kSlack, well inside
    // bf16/fp32 range.  scale > 0 makes the max of the raw scores, times the
    // scale, the max of the scaled scores.
    const bool need_mask = (key0 + kBN > kv_end) || (causal && key0 + kBN - 1 > C + q0 + wave * 32);
    u32x4_t pf[4];
    float psum = 0.0f;
    float alpha = 1.0f;
    bool rescale = false;   // wave-uniform; the accumulator is scaled after the branch
    auto update = [&](auto masked_tag) {
      constexpr bool kMasked = decltype(masked_tag)::value;
      if constexpr (kMasked) {
        // key = key0 + 4 (l / 32) + c with a compile-time c per register:
        // visible iff c <= lim (one compare per score)
        const int lim = (causal ? min(kv_end - 1, row_abs) : kv_end - 1) - key0 - 4 * (lane >> 5);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = hh * 32 + 8 * (i >> 2) + (i & 3);
            s[hh][i] = c <= lim ? s[hh][i] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[hh][i]);
      tmax = fmaxf(tmax, lane_xor(tmax, 32));
      const float tm = tmax == -INFINITY ? -INFINITY : tmax * scale2;
      if (__any(tm > m_run + kSlack)) {
        const float m_new = fmaxf(m_run, tm);
        alpha = fast_exp2(m_run - m_new);
        rescale = true;
        m_run = m_new;
        l_run *= alpha;
      }
      // P^T in bf16, packed as the B operand: regs 8 st .. 8 st + 7 of half hh
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = s[hh][8 * st + j];
            const float e = fast_exp2(fmaf(x, scale2, -m_run));
            p[j] = kMasked ? (x == -INFINITY ? 0.0f : e) : e;
            psum += p[j];
          }
          pf[2 * hh + st] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        }
      l_run += psum;
    };
    if (need_mask) update(std::true_type{});
    else update(std::false_type{});
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    }

    // O^T += V^T P^T: 4 key steps of 16 x 4 d tiles of 32.  Lane gi of
    // 16-lane group grp reads 4 bf16 of key row 16 ks + vr0 (+8) at dims
    // 32 dt + 16 (grp % 2) + 4 (gi % 4): chunk 4 dt + c0, half gi % 2, with
    // c0 = 2 (grp % 2) + (gi % 4)/2, in slot (4 dt + c0) ^ swz(row): one base
    // per (dt, row vr0 or vr0 + 8); 16 ks rows further is a constant offset.
    const int grp = lane >> 4;              // 16-lane group
    const int gi = lane & 15;
    const int kg = lane >> 5;               // k group
    const int c0 = 2 * (grp & 1) + ((gi & 3) >> 1);
    const int vr0 = 4 * kg + (gi >> 2);     // key row within a 16-key step, < 8
    const char* vb[2][4];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vb[e][dt] = vt + (vr0 + 8 * e) * kRowBytes + 16 * ((4 * dt + c0) ^ swz(vr0 + 8 * e)) + 8 * (gi & 1);
    // (ks, dt) steps in order, the two reads of a step issued kVD steps ahead
    constexpr int kVD = 4;
    u32x2_t vr[kVD + 1][2];
    auto vissue = [&](auto ic) {
      constexpr int i = decltype(ic)::value, ks = i / 4, dt = i % 4, b = i % (kVD + 1);
      vr[b][0] = lds_read_tr_issue<16 * ks * kRowBytes>(vb[0][dt]);
      vr[b][1] = lds_read_tr_issue<16 * ks * kRowBytes>(vb[1][dt]);
    };
    static_for<kVD>([&](auto ic) { vissue(ic); });
    static_for<16>([&](auto ic) {
      constexpr int i = decltype(ic)::value, ks = i / 4, dt = i % 4, b = i % (kVD + 1);
      if constexpr (i + kVD < 16) vissue(std::integral_constant<int, i + kVD>{});
      constexpr int kLater = 2 * (i + kVD < 16 ? kVD : 15 - i);
      lds_wait<kLater>(vr[b][0], vr[b][1]);
      const u32x2_t v1 = vr[b][0], v2 = vr[b][1];
      const u32x4_t vf = u32x4_t{v1.x, v1.y, v2.x, v2.y};
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), acc[dt], 0, 0, 0);
    });

    if (t + 1 < n_tiles) {
      if constexpr (kFp8) {
        // every wave is done reading the tile buffer; then tile t + 1's
        // widened codes go in, and the second barrier publishes them
        __syncthreads();
        rstore(smem);
        __syncthreads();
      } else {
        // this wave's loads of tile t + 1 have landed; after the barrier every
        // wave's have, and every wave is done reading buffer buf (its LDS reads
        // were waited for), which the loads issued at the start of iteration
        // t + 1 refill.  A bare barrier: the tiles' only writer is the DMA.
        gwait();
        __builtin_amdgcn_s_barrier();
      }
    }
  }

  // ---- finish: full row sum, normalise, write
  const float l_tot = l_run + lane_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? (kFp8 ? a.v_scale : 1.0f) / l_tot : 0.0f;
  if constexpr (kPrefix) {
    const int64_t prow = (int64_t(split) * a.num_tokens + my_row / G) * Hq + h;
    float* po = a.part_o + prow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * (lane >> 5);
        *reinterpret_cast<f32x4_t*>(po + d) =
            f32x4_t{acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv,
                    acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv};
      }
    if (lane < 32)
      a.part_lse[prow] = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    return;
  }
  const int64_t orow = int64_t(q_start) + my_row;
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

// ---------------------------------------------------------------------------
// Ping-pong varlen prefill (bf16 cache): the tiling and arithmetic of
// prefill_kernel<false, false>, laid out for gfx950's issue rules.
//
// A wave that is issuing MFMAs on gfx950 can slot in only about two VALU
// instructions per 32-cycle v_mfma_f32_32x32x16_bf16, while a second wave on
// the same SIMD issues VALU at nearly its full rate meanwhile.  So the
// softmax of one wave should run while another wave's MFMAs occupy the
// matrix unit.  A work-group of 8 waves owns 256 query rows of one query
// head: group 0 (waves 0-3) rows 0-127, group 1 (waves 4-7) rows 128-255,
// wave w4 of a group 32 rows; waves w and w + 4 share a SIMD.  Both groups
// walk the same 64-key tiles, half a period apart: in half-period h the group
// whose parity matches h issues its MFMAs -- O += P V of its previous tile,
// then S = Q K^T of its current one -- while the other group turns the scores
// it computed in h - 1 into P (online softmax, rescale of its output) and
// gathers tiles for later.  A barrier ends each half-period.
//
// Tiles: K of tile t lives in K slot t % (kLead + 1), V in V slot t % (kLead + 1)
// (16 KiB each, prefill_kernel's swizzled rows).  Group 0 reads K(p) and
// V(p - 1) in half-period 2p, group 1 in 2p + 1.  Group 1 gathers K(p + kLead)
// in half-period 2p, group 0 V(p + kLead - 1) in 2p + 1 (global_load_lds, four
// 1 KiB loads per wave): every tile is fetched into LDS once for both
// groups, sixteen loads per half-period per compute unit.  A slot is refilled
// only after the barrier that ends the last half-period reading it.  At the
// end of each half-period every wave waits for its own loads issued two or
// more half-periods earlier, and the barrier makes everybody's visible.  Page
// ids come from the block table by scalar loads issued two half-periods
// before the gather that uses them; the page of a key is a multiply-high by
// a reciprocal of the block size (exact for keys below 2^32 / block_size,
// which the host checks).  Blocks are aligned to the end of each request's
// chunk, so that a partial block holds its first rows, which see the fewest
// keys.

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt not waited for)
template <int N>
constexpr int vmcnt_imm() { return (N & 15) | ((N >> 4) << 14) | 0x0F70; }

constexpr int kPPRows = 256;   // query rows per ping-pong work-group
constexpr int kPD = 7;          // fused MFMA stream: LDS reads issued this many MFMAs ahead
constexpr int kPtabGroups = 4096;   // 16-key groups of the ping-pong kernel's address table

// LDS reads issued for MFMAs first..last of the fused stream (S's 16 MFMAs
// read one fragment each, PV's 16 two each)
constexpr int fused_reads_between(int first, int last) {
  int n = 0;
  for (int j = first; j <= last && j < 32; ++j) n += j < 16 ? 1 : 2;
  return n;
}
static_assert(fused_reads_between(1, kPD - 1) + 2 <= 15, "LDS reads in flight must fit lgkmcnt");

template <int kLead>   // load lead in periods; kLead + 1 K slots and kLead + 1 V slots
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(PrefillVarlen a) {
  static_assert(kLead >= 2, "the wait rule needs two half-periods of lead");
  constexpr int kSlots = kLead + 1;
  static_assert(2 * kSlots * kTileBytes + 8 * (kPtabGroups + 4) <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) char smem[2 * kSlots * kTileBytes];   // K slots, then V slots
  __shared__ __align__(16) uint64_t ptab[kPtabGroups + 4];       // 16-key group addresses
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();        // 0..7
  const int grp = wave >> 2;         // 0: rows 0-127 of the block, 1: rows 128-255
  const int w4 = wave & 3;
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int bs = a.block_size;
  const int id = blockIdx.x;
  const int xcd = id % kXcds;
  const int slot = id / kXcds;

  // work-group -> (request, KV head, q block, head of the group): every q
  // block and query head of one (request, KV head) pair on one XCD, one after
  // another (their K/V is read from HBM once and then from that XCD's L2),
  // the block with the most keys (the chunk's last rows) first
  const int n_qb = (a.max_query_len + kPPRows - 1) / kPPRows;
  const int per_pair = n_qb * G;
  const int pair = (slot / per_pair) * kXcds + xcd;
  if (pair >= a.num_seqs * a.num_kv_heads) return;
  const int local = slot % per_pair;
  const int r = pair / a.num_kv_heads;
  const int kvh = pair % a.num_kv_heads;
  const int qb = local / G;          // 0: the chunk's last kPPRows rows
  const int h = kvh * G + local % G;
  const int q_start = min(max(a.query_start_loc[r], 0), a.num_tokens);
  const int L = min(min(a.query_start_loc[r + 1] - q_start, a.max_query_len), a.num_tokens - q_start);
  const int S = min(a.seq_lens[r], a.max_blocks * bs);
  const int qend = L - qb * kPPRows;   // block rows [qend - 256, qend) of the chunk
  if (L <= 0 || qend <= 0) return;
  const int C = S - L;
  const bool causal = a.causal != 0;
  auto group_end = [&](int g) __attribute__((always_inline)) {   // keys rows qend - 256 + 128 g .. + 127 may see
    const int last = qend - kPPRows + 128 * g + 127;
    if (last < 0) return 0;   // the group has no row
    return causal ? min(S, max(0, C + last + 1)) : S;
  };
  const int kv_end = group_end(1);     // the block's keys
  const int kv_mine = group_end(grp);  // this group's
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int n_mine = (kv_mine + kBN - 1) / kBN;

  // ---- Q fragments (B operand of S^T): row = l % 32, d chunk = 16 kk + 8 (l / 32)
  const int row0 = qend - kPPRows + 128 * grp + 32 * w4;   // this wave's first row
  const int my_row = row0 + (lane & 31);
  const bool row_ok = my_row >= 0;
  u32x4_t qf[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (int64_t(q_start) + (row_ok ? my_row : 0)) * Hq * kD + int64_t(h) * kD +
                         8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = row_ok ? load16(qp + 16 * kk) : u32x4_t{0, 0, 0, 0};
  }

  // ---- gathers: a plane (K or V) of a tile is 16 wave-wide 1 KiB loads,
  // wave w4 of the gathering group issuing loads j = w4 + 4 jj, jj = 0..3.
  // Load j fills rows 4 j .. 4 j + 3 (lane i: row 4 j + i / 16, slot i % 16,
  // which holds chunk slot ^ swz(row)); the rows of a load share one 16-key
  // group, jj, and so one page.  The address of every 16-key group of the
  // block's keys (page base plus the group's row in the page, K plane) is
  // put in LDS once, at the start: a load's address is then one table entry
  // plus a per-lane offset (two VALU adds), with no block-table read and no
  // scalar arithmetic in the loop.  The host sends sequences longer than the
  // table elsewhere.
  const int64_t tok_bytes = int64_t(a.num_kv_heads) * kD * 2;
  const char* cache_h = static_cast<const char*>(a.cache) + int64_t(kvh) * kD * 2;
  const int32_t* table = a.block_table + int64_t(r) * a.max_blocks;
  const uint32_t tok32 = uint32_t(tok_bytes);
  const uint32_t page_bytes = 2u * uint32_t(bs) * tok32;
  const uint32_t kv32 = uint32_t(bs) * tok32;
  const uint32_t nblk = uint32_t(min(a.num_blocks, int64_t(INT32_MAX)));
  const int last16 = ((kv_end - 1) / 16) * 16;
  const int ng = last16 / 16 + 1;   // 16-key groups of the block's keys, <= kPtabGroups
  for (int g = threadIdx.x; g < ng + 4; g += 512) {   // four copies of the last past the end
    const int key16 = 16 * min(g, ng - 1);
    const int page = key16 / bs;
    uint32_t blk = uint32_t(table[page]);
    blk = blk < nblk ? blk : 0u;   // negative ids wrap high
    ptab[g] = reinterpret_cast<uint64_t>(cache_h) + uint64_t(blk) * page_bytes +
              uint32_t(key16 - page * bs) * tok32;
  }
  const int plane = grp == 0 ? 0 : 1;   // group 0 gathers K, group 1 V
  const uint32_t plane_off = plane ? kv32 : 0u;
  // byte offset of this lane's 16 bytes from its 16-key group's first row
  // (the same for every jj: row % 16 = 4 w4 + lane / 16), plus the plane
  const int lrow = 4 * w4 + (lane >> 4);
  const uint32_t my_off = uint32_t(lrow * tok_bytes + 16 * ((lane & 15) ^ swz(lrow))) + plane_off;
  // the four group addresses of a tile (tiles outside [0, n_tiles) read the
  // last: in bounds, never used)
  auto ptab_read = [&](int tile, uint64_t (&pt)[4]) {
    const int g0 = 4 * min(max(tile, 0), n_tiles - 1);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) pt[jj] = ptab[g0 + jj];
  };
  // load jj of a tile; keys past kv_end re-read key kv_end - 1
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue = [&](int tile, const uint64_t (&pt)[4], int jj, int slot) {
    uint32_t off = my_off;
    if (tile * kBN + kBN > kv_end) {   // wave-uniform
      const int key16 = min(tile * kBN + 16 * jj, last16);
      off = uint32_t(min(lrow, kv_end - 1 - key16) * tok_bytes + 16 * ((lane & 15) ^ swz(lrow))) +
            plane_off;
    }
    char* dst = smem + (plane * kSlots + slot) * kTileBytes + 1024 * (w4 + 4 * jj);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(pt[jj]) + off, (lds_ptr)dst, 16, 0, 0);
  };
  auto gather = [&](int tile, const uint64_t (&pt)[4]) {   // the four loads back to back
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) issue(tile, pt, jj, tile % kSlots);
  };

  const float scale2 = a.scale * kLog2e;
  float m_run = kNoMax;   // running max (base-2 domain) of row my_row
  float l_run = 0.0f;     // this lane's share of the running sum
  f32x16_t acc[4];        // O^T tiles: d = 32 dt + 8 (r/4) + 4 (l/32) + r%4
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  f32x16_t s[2];          // S^T of the group's current tile
  u32x4_t pf[4] = {};     // P^T (bf16) of the group's previous tile (zero: none)
  const int row_abs = C + my_row;

  // S^T = K Q^T for tile t (two 32-key halves, LDS reads two k-steps ahead).
  // kaddr[kk]: this lane's chunk of k-step kk in K slot 0 (row l % 32, chunk
  // 2 kk + l / 32 in slot (chunk ^ swz(row))); the second half is 32 rows on.
  const uint32_t smem_base = lds_addr(smem);
  uint32_t kaddr[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    kaddr[kk] = smem_base + (lane & 31) * kRowBytes + 16 * ((2 * kk + (lane >> 5)) ^ swz(lane & 31));
  auto scores = [&](int t) __attribute__((always_inline)) {
    const uint32_t kslot = uint32_t(t % kSlots) * kTileBytes;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[hh][i] = 0.0f;
    constexpr int kQD = 2;
    u32x4_t kr[kQD + 1][2];
    auto kissue = [&](auto kc) __attribute__((always_inline)) {
      constexpr int kk = decltype(kc)::value, b = kk % (kQD + 1);
      const uint32_t ad = kaddr[kk] + kslot;
      kr[b][0] = lds_read16_at<0>(ad);
      kr[b][1] = lds_read16_at<32 * kRowBytes>(ad);
    };
    static_for<kQD>([&](auto kc) __attribute__((always_inline)) { kissue(kc); });
    static_for<8>([&](auto kc) __attribute__((always_inline)) {
      constexpr int kk = decltype(kc)::value, b = kk % (kQD + 1);
      if constexpr (kk + kQD < 8) kissue(std::integral_constant<int, kk + kQD>{});
      constexpr int kLater = 2 * (kk + kQD < 8 ? kQD : 7 - kk);
      lds_wait<kLater>(kr[b][0], kr[b][1]);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[b][0]), as_bf16x8(qf[kk]), s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[b][1]), as_bf16x8(qf[kk]), s[1], 0, 0, 0);
    });
  };

  // O^T += V^T P^T for tile t (4 key steps x 4 d tiles, reads four steps
  // ahead).  Lane gi of 16-lane group vg reads 4 bf16 of key row 16 ks + vr0
  // (+ 8) at dims 32 dt + 16 (vg % 2) + 4 (gi % 4): chunk 4 dt + c0 in slot
  // (4 dt + c0) ^ swz(row); 16 ks rows further is an immediate offset.
  uint32_t vaddr[2][4];
  {
    const int vg = lane >> 4, gi = lane & 15, kg = lane >> 5;
    const int c0 = 2 * (vg & 1) + ((gi & 3) >> 1);
    const int vr0 = 4 * kg + (gi >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vaddr[e][dt] = smem_base + kSlots * kTileBytes + (vr0 + 8 * e) * kRowBytes +
                       16 * ((4 * dt + c0) ^ swz(vr0 + 8 * e)) + 8 * (gi & 1);
  }
  auto pv = [&](int t) __attribute__((always_inline)) {
    const uint32_t vslot = uint32_t(t % kSlots) * kTileBytes;
    constexpr int kVD = 4;
    u32x2_t vr[kVD + 1][2];
    auto vissue = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, ks = i / 4, dt = i % 4, b = i % (kVD + 1);
      vr[b][0] = lds_read_tr_at<16 * ks * kRowBytes>(vaddr[0][dt] + vslot);
      vr[b][1] = lds_read_tr_at<16 * ks * kRowBytes>(vaddr[1][dt] + vslot);
    };
    static_for<kVD>([&](auto ic) __attribute__((always_inline)) { vissue(ic); });
    static_for<16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, ks = i / 4, dt = i % 4, b = i % (kVD + 1);
      if constexpr (i + kVD < 16) vissue(std::integral_constant<int, i + kVD>{});
      constexpr int kLater = 2 * (i + kVD < 16 ? kVD : 15 - i);
      lds_wait<kLater>(vr[b][0], vr[b][1]);
      const u32x2_t v1 = vr[b][0], v2 = vr[b][1];
      const u32x4_t vf = u32x4_t{v1.x, v1.y, v2.x, v2.y};
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), acc[dt], 0, 0, 0);
    });
  };

  // online softmax of tile t's scores (see prefill_kernel): P^T into pf,
  // the running max / sum, and the output's rescale.  Not live (no tile to
  // process: before the first, past the group's last) it masks every score,
  // which leaves the row state as it is and P zero, so that the following
  // PV MFMAs add nothing.
  auto softmax = [&](int t, bool live) __attribute__((always_inline)) {
    const int key0 = t * kBN;
    const bool need_mask = !live || (key0 + kBN > kv_mine) || (causal && key0 + kBN - 1 > C + row0);
    float psum = 0.0f;
    float alpha = 1.0f;
    bool rescale = false;   // wave-uniform
    auto update = [&](auto masked_tag) __attribute__((always_inline)) {
      constexpr bool kMasked = decltype(masked_tag)::value;
      if constexpr (kMasked) {
        const int lim = live ? (causal ? min(kv_mine - 1, row_abs) : kv_mine - 1) - key0 - 4 * (lane >> 5)
                             : -1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = hh * 32 + 8 * (i >> 2) + (i & 3);
            s[hh][i] = c <= lim ? s[hh][i] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[hh][i]);
      tmax = xor32_max(tmax);
      const float tm = tmax == -INFINITY ? -INFINITY : tmax * scale2;
      if (__any(tm > m_run + kSlack)) {
        const float m_new = fmaxf(m_run, tm);
        alpha = fast_exp2(m_run - m_new);
        rescale = true;
        m_run = m_new;
        l_run *= alpha;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = s[hh][8 * st + j];
            const float e = fast_exp2(fmaf(x, scale2, -m_run));
            p[j] = kMasked ? (x == -INFINITY ? 0.0f : e) : e;
            psum += p[j];
          }
          pf[2 * hh + st] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        }
      l_run += psum;
    };
    if (need_mask) update(std::true_type{});
    else update(std::false_type{});
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
    }
  };

  // ---- gathers: the group issuing MFMAs in a half-period also issues that
  // half-period's gather, between its MFMAs (a wave's MFMA leaves it free
  // issue cycles, while the softmax wave is bound by its own VALU and scalar
  // instructions).  Group 0 gathers K(h / 2 + kLead) in even h, group 1
  // V((h - 1) / 2 + kLead - 1) in odd h; each keeps the page ids of its
  // next tile, fetched at the end of its previous gather half-period.
  auto my_tile = [&](int h) __attribute__((always_inline)) {   // the tile this wave gathers in half-period h, or -1
    if (grp == 0 && (h & 1) == 0) return h / 2 + kLead;
    if (grp == 1 && (h & 1) != 0) return (h - 1) / 2 + kLead - 1;
    return -1;
  };
  auto n_issued = [&](int h) __attribute__((always_inline)) {
    const int t = my_tile(h);
    return t >= 0 && t < n_tiles ? 4 : 0;
  };
  // after half-period hp the loads of hp - 1 and hp may stay in flight
  auto wait_loads = [&](int hp) __attribute__((always_inline)) {
    const int later = n_issued(hp) + n_issued(hp - 1);
    if (later >= 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm<4>());
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  };

  // ---- prologue: zeros into the V slots (read, times a zero P, before any
  // V lands in them) and the address table published, then the gathers of
  // half-periods -2 kLead .. -1; K(0) has landed for every wave after the
  // barrier.  pt holds the group addresses of this wave's next gather.
  for (int i = threadIdx.x; i < kSlots * kTileBytes / 16; i += 512)
    *reinterpret_cast<u32x4_t*>(smem + kSlots * kTileBytes + 16 * i) = u32x4_t{0, 0, 0, 0};
  __syncthreads();
  uint64_t pt[4];
  for (int hh = -2 * kLead; hh < 0; ++hh) {
    const int t = my_tile(hh);
    if (t >= 0 && t < n_tiles) {
      ptab_read(t, pt);
      gather(t, pt);
    }
  }
  ptab_read(my_tile(grp == 0 ? 0 : 1), pt);
  wait_loads(-1);
  __builtin_amdgcn_s_barrier();

  // The MFMA block of a half-period: S(p) and PV(p - 1) as one stream of 32
  // MFMAs (S's 16, then PV's 16) whose LDS reads run kPD MFMAs ahead across
  // the two (a wave's LDS reads take over a hundred cycles to land), with
  // the gather's four loads between them.  K(p) has landed a half-period
  // before the block, so its first kPD - 1 reads go out at the end of the
  // wave's softmax half-period (kpre), before the barrier, right after the
  // table entries in pt are made to have landed (they were read a
  // half-period before; the compiler, which does not see the stream's LDS
  // reads, would wait for them with a wait for every LDS read in flight).
  // Without a PV to
  // do P is zero (V slots hold zeros or gathered keys, never NaN); without
  // an S to do (the last tile, or a group past its last tile, which still
  // gathers for the other) the scores are computed and dropped.  One path
  // for all cases: separate paths made the compiler keep the accumulators
  // twice.
  // The loops below are unrolled by the slot count, so that the slots a
  // period uses are compile-time constants (rc = p % kSlots) and every LDS
  // address is a per-lane base plus an immediate.
  u32x4_t kr[kPD];
  auto kread = [&](auto rc, auto ic) __attribute__((always_inline)) {   // K read of stream step i < 16 into kr
    constexpr int R = decltype(rc)::value, i = decltype(ic)::value, kk = i / 2, hh = i % 2;
    kr[i % kPD] = lds_read16_at<R * kTileBytes + 32 * kRowBytes * hh>(kaddr[kk]);
  };
  auto kpre = [&](auto rc) __attribute__((always_inline)) {
    asm volatile("" : "+v"(pt[0]), "+v"(pt[1]), "+v"(pt[2]), "+v"(pt[3]));
    static_for<kPD - 1>([&](auto ic) __attribute__((always_inline)) { kread(rc, ic); });
  };
  auto fused = [&](auto rc, int gt, bool go) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    constexpr int RV = (R + kSlots - 1) % kSlots;   // V slot of tile p - 1
    // the slot this wave's gather fills: K(p + kLead) or V(p + kLead - 1)
    const int gslot = plane == 0 ? (R + kLead) % kSlots : (R + kLead - 1) % kSlots;
    u32x2_t vr[kPD][2];
    auto rd = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, b = i % kPD;
      if constexpr (i < 16) {
        kread(rc, ic);
      } else {
        constexpr int ks = (i - 16) / 4, dt = (i - 16) % 4;
        constexpr int off = RV * kTileBytes + 16 * ks * kRowBytes;
        vr[b][0] = lds_read_tr_at<off>(vaddr[0][dt]);
        vr[b][1] = lds_read_tr_at<off>(vaddr[1][dt]);
      }
    };
    static_for<32>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, b = i % kPD;
      constexpr int kLater = fused_reads_between(i + 1, i + kPD - 1);
      if constexpr (i < 16) {
        constexpr int kk = i / 2, hh = i % 2;
        lds_wait1<kLater>(kr[b]);
        if constexpr (i + kPD - 1 < 32) rd(std::integral_constant<int, i + kPD - 1>{});
        s[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[b]), as_bf16x8(qf[kk]),
                                                        kk == 0 ? f32x16_t{} : s[hh], 0, 0, 0);
      } else {
        constexpr int ks = (i - 16) / 4, dt = (i - 16) % 4;
        lds_wait<kLater>(vr[b][0], vr[b][1]);
        if constexpr (i + kPD - 1 < 32) rd(std::integral_constant<int, i + kPD - 1>{});
        const u32x4_t vf = u32x4_t{vr[b][0].x, vr[b][0].y, vr[b][1].x, vr[b][1].y};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), acc[dt], 0, 0, 0);
      }
      if constexpr (i % 8 == 3) {   // load jj = i / 8
        if (go) issue(gt, pt, i / 8, gslot);
      }
    });
  };
  // One half-period of the group issuing MFMAs: S(p) and PV(p - 1) and this
  // wave's gather, then the table entries of its next gather (read after
  // the stream's last LDS wait, used a half-period later)
  auto mfma_half = [&](auto rc, int h) __attribute__((always_inline)) {
    const int gt = my_tile(h);
    const bool go = gt >= 0 && gt < n_tiles;   // wave-uniform
    fused(rc, gt, go);
    ptab_read(my_tile(h + 2), pt);
  };
  auto end_half = [&](int hp) __attribute__((always_inline)) {
    wait_loads(hp);
    __builtin_amdgcn_s_barrier();
  };
  // Each group runs its own loop, so that its two blocks follow each other
  // in straight-line code.
  if (grp == 0) {
    kpre(std::integral_constant<int, 0>{});
    for (int p = 0; p <= n_tiles;) {
      static_for<kSlots>([&](auto rc) __attribute__((always_inline)) {
        if (p <= n_tiles) {
          constexpr int R = decltype(rc)::value;
          mfma_half(rc, 2 * p);                // half-period 2p
          end_half(2 * p);
          softmax(p, p < n_mine);              // half-period 2p + 1
          kpre(std::integral_constant<int, (R + 1) % kSlots>{});
          end_half(2 * p + 1);
          ++p;
        }
      });
    }
  } else {
    for (int p = 0; p <= n_tiles;) {
      static_for<kSlots>([&](auto rc) __attribute__((always_inline)) {
        if (p <= n_tiles) {
          softmax(p - 1, p >= 1 && p - 1 < n_mine);   // half-period 2p
          kpre(rc);
          end_half(2 * p);
          mfma_half(rc, 2 * p + 1);            // half-period 2p + 1
          end_half(2 * p + 1);
          ++p;
        }
      });
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the last kpre's reads, unused

  // ---- finish: full row sum, normalise, write
  const float l_tot = xor32_sum(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int64_t orow = int64_t(q_start) + my_row;
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
  if (a.prefix_splits > 0) {
    if (a.num_tokens <= 0 || a.prefix_len <= 0) return hipSuccess;
    if (a.split_keys <= 0 || a.split_keys % kBN != 0) return hipErrorInvalidValue;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int64_t n_qt = (int64_t(a.num_tokens) * G + kBM - 1) / kBM;
    const int64_t pairs = int64_t(a.num_kv_heads) * a.prefix_splits;
    const int64_t wgs = (pairs + kXcds - 1) / kXcds * kXcds * n_qt;
    if (wgs > INT32_MAX || int64_t(a.num_tokens) * G > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<true, false>), dim3(unsigned(wgs)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.num_seqs <= 0 || a.num_tokens <= 0 || a.max_query_len <= 0) return hipSuccess;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t pairs = int64_t(a.num_seqs) * a.num_kv_heads;
  if (a.fp8) {
    const int n_qt = (a.max_query_len + kBM - 1) / kBM;
    const int64_t wgs = (pairs + kXcds - 1) / kXcds * kXcds * n_qt * G;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<false, true>), dim3(unsigned(wgs)), dim3(256), 0, s, a);
  } else {
    if (int64_t(a.max_blocks) * a.block_size <= 16 * int64_t(kPtabGroups)) {
      const int n_qb = (a.max_query_len + kPPRows - 1) / kPPRows;
      const int64_t wgs = (pairs + kXcds - 1) / kXcds * kXcds * n_qb * G;
      if (wgs > INT32_MAX) return hipErrorInvalidValue;
      hipLaunchKernelGGL(prefill_pp_kernel<kPrefillLead>, dim3(unsigned(wgs)), dim3(512), 0, s, a);
    } else {   // keys beyond the ping-pong kernel's address table
      const int n_qt = (a.max_query_len + kBM - 1) / kBM;
      const int64_t wgs = (pairs + kXcds - 1) / kXcds * kXcds * n_qt * G;
      if (wgs > INT32_MAX) return hipErrorInvalidValue;
      hipLaunchKernelGGL((prefill_kernel<false, false>), dim3(unsigned(wgs)), dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace pa
