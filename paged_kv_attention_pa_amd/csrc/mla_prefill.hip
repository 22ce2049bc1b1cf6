// MLA prefill in the multi-head form over the latent cache.
//
// Method: "Triton 與 MLA：可移植注意力與潛空間注意力" (設計動機, 關鍵檔案: the MLA
// layer holds kv_b_proj, qk_nope_head_dim, qk_rope_head_dim and kv_lora_rank;
// its backend's prefill entry point is the multi-head form) and "Attention
// Backends" (latent attention: prefill and decode use different formulations
// of the same mathematics).  Per head h the key of position j is
// [W_k[h] kv_c_j | k_pe_j] (128 + 64) and its value W_v[h] kv_c_j (128), with
// kv_b_proj's weight W [H, 256, 512] (rows 0..127 of a head expand keys, rows
// 128..255 values); causal attention of the chunk's queries [q_nope | q_pe]
// ("第 1 章 注意力后端", §2.1, bottom-right aligned; §4.1 tiling with an
// online softmax).
//
// Three kernels:
// * mla_schedule_kernel: cumulative key counts of the requests (one block
//   scan), then the attention's work list: every (request, 128-query tile)
//   item, requests longest first (counting sort on the key tiles of their last
//   q tile), a request's q tiles together and longest first, so that the long
//   items start early, the short ones fill the tail, and the q tiles sharing
//   keys run close together.
// * mla_expand_kernel: the projection of every key of the batch, a bf16 GEMM
//   E^T[n][g] = sum_k W[n][k] L[g][k] over the gathered latent rows L (n = a
//   projection output of one head, g = a key of the batch), 128 x 256 tiles on
//   v_mfma_f32_32x32x16_bf16, both operands staged in LDS by
//   global_load_lds_dwordx4 (32-deep k slices in a three-stage ring, two
//   work-groups per CU); the work-group holding a head's key rows also copies
//   k_pe next to them, so the expanded key row is 192 contiguous elements.
// * mla_attn_kernel: the prefill kernel's tiling (128 query rows of one head
//   per work-group, 64-key tiles gathered into LDS by DMA, S^T = K Q^T and
//   O^T += V^T P^T on 32x32x16 MFMAs, online softmax in the exp2 domain) with
//   a 192-wide key (a 128-wide tile and a 64-wide rope tile) read from the
//   expanded rows, which are contiguous per request.
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kR = 512;          // kv_lora_rank
constexpr int kP = 64;           // rope dims
constexpr int kDn = 128;         // qk_nope dims
constexpr int kDv = 128;         // v dims
constexpr int kDq = kDn + kP;    // 192: query / key width
constexpr int kLatBytes = (kR + kP) * 2;   // 1152 B per latent row
constexpr int kXcds = 8;

// ------------------------------------------------------------- expansion
constexpr int kEM = 128;                     // projection outputs per work-group
constexpr int kEN = 256;                     // keys per work-group
constexpr int kEK = 32;                      // k per stage
constexpr int kESlice = kEK * 2;             // 64 B of a row per stage
constexpr int kEWTile = kEM * kESlice;       // 8 KiB of W per stage
constexpr int kELTile = kEN * kESlice;       // 16 KiB of latent rows per stage
constexpr int kEStage = kEWTile + kELTile;   // 24 KiB
constexpr int kERing = 3;                    // stages in LDS: two in flight
// ring layout: the three W slices first, then the three latent slices
constexpr int kELBase = kERing * kEWTile;
constexpr int kESteps = kR / kEK;            // 16 stages over kv_lora_rank
constexpr int kEWLoads = kEWTile / 1024 / 4; // wave-wide 16-byte loads per wave and stage: W
constexpr int kELoads = kEStage / 1024 / 4;  // all (W first)
// 16-byte chunk c (0..3) of row r of a staged slice sits in slot
// c ^ ((r >> 2) & 3): rows are 64 B, so a 16-lane phase reading one chunk of
// 16 consecutive rows hits 16 distinct 16-byte bank groups.
__device__ __forceinline__ int eslot(int r, int c) { return c ^ ((r >> 2) & 3); }

// Two work-groups per CU (74 KiB of LDS each): one's prologue (row lookup,
// first loads) and epilogue (the stores of its outputs) run under the other's
// MFMA work.
__global__ __launch_bounds__(256, 2) void mla_expand_kernel(MlaPrefill a) {
  __shared__ __align__(16) char smem[kERing * kEStage];
  __shared__ uint64_t s_row[kEN];             // byte offset of each key's latent row
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int H = a.num_heads;
  const int n_tiles = 2 * H;                  // a tile is the key half or the value half of a head
  // XCD-aware order.  When the n tiles divide over the XCDs, XCD x keeps a
  // quarter of W (n group x % 4) in its L2 and walks half of the key tiles
  // (x / 4): each latent row is fetched by 4 XCDs, and W plus the latent
  // tiles in flight fit the 4 MiB L2.  Otherwise the n tiles of one key tile
  // run on one XCD, one after another, and share its latent rows there.
  const int id = blockIdx.x;
  const int xcd = id % kXcds, slot = id / kXcds;
  int g_tile, n_tile;
  if (n_tiles % kXcds == 0) {
    const int n_per = n_tiles / 4;            // 4 groups of n tiles x 2 halves of the key tiles
    n_tile = (xcd & 3) * n_per + slot % n_per;
    g_tile = (slot / n_per) * 2 + (xcd >> 2);
  } else {
    g_tile = (slot / n_tiles) * kXcds + xcd;
    n_tile = slot % n_tiles;
  }
  const int total = a.total_keys;
  const int g0 = g_tile * kEN;
  if (g0 >= total) return;
  const int h = n_tile >> 1, half = n_tile & 1;

  // latent row of each key of the tile (keys past the batch re-read the last)
  {
    const int g = min(g0 + tid, total - 1);
    int lo = 0, hi = a.num_seqs - 1;          // request r with key_start[r] <= g < key_start[r + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.key_start[mid] <= g) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int j = g - a.key_start[r];
    const int page = j / a.block_size;
    int64_t blk = a.block_table[int64_t(r) * a.max_blocks + page];
    blk = (blk < 0 || blk >= a.num_blocks) ? 0 : blk;
    s_row[tid] = uint64_t((blk * a.block_size + (j - page * a.block_size)) * int64_t(kLatBytes));
  }
  __syncthreads();

  const char* wbase = static_cast<const char*>(a.w) + int64_t(n_tile) * kEM * (kR * 2);
  const char* cbase = static_cast<const char*>(a.cache);
  // DMA: a stage is 24 wave-wide loads of 16 rows x 64 B: loads 0..7 the W
  // slice, 8..23 the latent slice; wave w issues loads j = w + 4 jj (its
  // first two are W loads).  Lane i of load j: row 16 j' + i / 4 of its
  // operand (j' = j, or j - 8), slot i % 4, which holds chunk eslot(row, slot).
  constexpr int kWJ = 4 * kEWLoads;   // W loads per stage
  const char* src[kELoads];   // this lane's bytes of each of its loads (stage 0)
#pragma unroll
  for (int jj = 0; jj < kELoads; ++jj) {
    const int j = wave + 4 * jj;
    if (jj < kEWLoads) {
      const int row = 16 * j + (lane >> 2);
      src[jj] = wbase + row * (kR * 2) + 16 * eslot(row, lane & 3);
    } else {
      const int row = 16 * (j - kWJ) + (lane >> 2);
      src[jj] = cbase + s_row[row] + 16 * eslot(row, lane & 3);
    }
  }
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto gload = [&](int stage) {
    const int slot = stage % kERing;
#pragma unroll
    for (int jj = 0; jj < kELoads; ++jj) {
      const int j = wave + 4 * jj;
      char* dst = jj < kEWLoads ? smem + slot * kEWTile + 1024 * j
                                : smem + kELBase + slot * kELTile + 1024 * (j - kWJ);
      __builtin_amdgcn_global_load_lds(src[jj] + stage * kESlice, (lds_ptr)dst, 16, 0, 0);
    }
  };

  // wave tile: all 128 outputs x keys 64 w .. + 63 (4 x 2 MFMA tiles)
  const int c32 = lane & 31, kh = lane >> 5;
  f32x16_t acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][gi][i] = 0.0f;

  // LDS operand addresses of k-step kk (ring slot 0): output rows 32 mi + c32
  // of the W slice, key rows 64 wave + 32 gi + c32 of the latent slice, chunk
  // 2 kk + kh.  The reads are inline assembly with explicit waits: the
  // compiler cannot tell them apart from the DMA filling the other slots and
  // would wait for those loads first.
  constexpr int kKSteps = kEK / 16;
  uint32_t ra[kKSteps][4], rb[kKSteps][2];
  {
    const uint32_t base = lds_addr(smem);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = 32 * mi + c32;
        ra[kk][mi] = base + uint32_t(r * kESlice + 16 * eslot(r, 2 * kk + kh));
      }
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int r = 64 * wave + 32 * gi + c32;
        rb[kk][gi] = base + uint32_t(kELBase + r * kESlice + 16 * eslot(r, 2 * kk + kh));
      }
    }
  }
  gload(0);
  gload(1);
  static_for<kESteps>([&](auto sc) {
    constexpr int st = decltype(sc)::value;
    constexpr int kSlot = st % kERing;
    constexpr int kAOff = kSlot * kEWTile;
    constexpr int kBOff = kSlot * kELTile;
    static_assert(kAOff < 65536 && kBOff < 65536, "immediate LDS offsets");
    // stage st has landed for this wave when the loads of the stages issued
    // after it are the only ones outstanding
    static_assert(kELoads == 6, "the wait below counts one stage's loads");
    if constexpr (st + 1 < kESteps) __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                               // vmcnt(0)
    __builtin_amdgcn_s_barrier();   // everyone's loads of st; everyone done with st - 1
    if constexpr (st + 2 < kESteps) gload(st + 2);   // refills the slot of st - 1
    u32x4_t af[2][4], bf[2][2];     // [k-step parity][tile]
    auto issue = [&](auto kc) {
      constexpr int kk = decltype(kc)::value;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[kk & 1][mi] = lds_read16_at<kAOff>(ra[kk][mi]);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) bf[kk & 1][gi] = lds_read16_at<kBOff>(rb[kk][gi]);
    };
    issue(std::integral_constant<int, 0>{});
    static_for<kKSteps>([&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      if constexpr (kk + 1 < kKSteps) {
        issue(std::integral_constant<int, kk + 1>{});
        lds_wait<6>(af[kk & 1][0], af[kk & 1][1], af[kk & 1][2], af[kk & 1][3]);
        lds_wait<6>(bf[kk & 1][0], bf[kk & 1][1]);
      } else {
        lds_wait<0>(af[kk & 1][0], af[kk & 1][1], af[kk & 1][2], af[kk & 1][3]);
        lds_wait<0>(bf[kk & 1][0], bf[kk & 1][1]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
          acc[mi][gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(af[kk & 1][mi]), as_bf16x8(bf[kk & 1][gi]), acc[mi][gi], 0, 0, 0);
    });
  });

  // Epilogue through LDS (the ring is free: every stage has been read), so
  // that each key's 128 outputs leave as 256 contiguous bytes.  E^T tile
  // (mi, gi): lane l holds key g = 64 wave + 32 gi + l % 32 and outputs
  // n = 32 mi + 8 (i / 4) + 4 (l / 32) + i % 4, written to the staging row of
  // key g (272-byte rows: 256 B + 16 B of padding).
  constexpr int kORow = kEM * 2 + 16;
  static_assert(kEN * kORow <= kERing * kEStage, "epilogue staging fits the ring");
  // the key half also places k_pe after the head's 128 projected dims: its
  // loads go out first (keys past the batch read the last key's row)
  u32x4_t pe[8] = {};
  if (half == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i;          // 256 rows x 8 chunks of 16 B
      pe[i] = load16(cbase + s_row[q >> 3] + kR * 2 + 16 * (q & 7));
    }
  }
  __builtin_amdgcn_s_barrier();   // every wave is done reading the ring
  {
    const uint32_t base = lds_addr(smem);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int g = 64 * wave + 32 * gi + c32;
          const int n = 32 * mi + 8 * q4 + 4 * kh;
          u32x2_t v;
          v.x = pack_bf16x2(acc[mi][gi][4 * q4 + 0], acc[mi][gi][4 * q4 + 1]);
          v.y = pack_bf16x2(acc[mi][gi][4 * q4 + 2], acc[mi][gi][4 * q4 + 3]);
          asm volatile("ds_write_b64 %0, %1" : : "v"(base + uint32_t(g * kORow + 2 * n)), "v"(v) : "memory");
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  // the k_pe rows have arrived before any output store is issued (a wait
  // after those stores would wait for them too); unconditional, so that no
  // path reaches the k_pe stores with the loads still counted as pending
  asm volatile("s_waitcnt vmcnt(0)"
                 : "+v"(pe[0]), "+v"(pe[1]), "+v"(pe[2]), "+v"(pe[3]),
                   "+v"(pe[4]), "+v"(pe[5]), "+v"(pe[6]), "+v"(pe[7]));
  __builtin_amdgcn_s_barrier();
  const int64_t krow = int64_t(H) * kDq, vrow = int64_t(H) * kDv;   // elements per expanded row
  {
    // 256 keys x 16 chunks of 16 B: 16 per thread, 16 lanes per key row,
    // read four at a time
    const uint32_t base = lds_addr(smem);
    char* out = half == 0 ? static_cast<char*>(a.k_exp) + 2 * (int64_t(h) * kDq)
                          : static_cast<char*>(a.v_exp) + 2 * (int64_t(h) * kDv);
    const int64_t orow = 2 * (half == 0 ? krow : vrow);   // bytes per expanded row
#pragma unroll
    for (int i0 = 0; i0 < 16; i0 += 4) {
      u32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = tid + 256 * (i0 + u);
        v[u] = lds_read16_at<0>(base + uint32_t((q >> 4) * kORow + 16 * (q & 15)));
      }
      lds_wait<0>(v[0], v[1], v[2], v[3]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = tid + 256 * (i0 + u);
        const int g = g0 + (q >> 4);
        if (g < total)   // streaming stores: read back only after the whole projection
          __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(out + int64_t(g) * orow + 16 * (q & 15)));
      }
    }
  }
  if (half == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i;
      const int g = g0 + (q >> 3);
      if (g < total)
        __builtin_nontemporal_store(pe[i], reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.k_exp) + int64_t(g) * krow +
                                                                       int64_t(h) * kDq + kDn + 8 * (q & 7)));
    }
  }
}

// ------------------------------------------------------------- attention
constexpr int kBM = 128;                      // query rows per work-group
constexpr int kBN = 64;                       // keys per tile
constexpr int kNRow = kDn * 2;                // 256 B: key-nope and value rows
constexpr int kPRow = kP * 2;                 // 128 B: rope rows
constexpr int kNTile = kBN * kNRow;           // 16 KiB
constexpr int kPTile = kBN * kPRow;           // 8 KiB
constexpr int kAStage = 2 * kNTile + kPTile;  // K nope, V, K rope: 40 KiB
constexpr float kSlack = 8.0f;
// 256-byte rows: chunk c of row r in slot c ^ swz(r) (16 slots, as in the
// varlen prefill kernel: conflict-free K-fragment and V^T reads); 128-byte
// rope rows: slot c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int pslot(int r, int c) { return c ^ ((r >> 1) & 7); }

// Request r's queries [q_start, q_start + L) and keys [ks, ks + S) of the
// expanded buffers, clamped to the rows that exist (the schedule and the
// attention read them through this one function).
struct ReqGeom { int q_start, L, ks, S; };
__device__ __forceinline__ ReqGeom request_geometry(const MlaPrefill& a, int r) {
  ReqGeom g;
  g.q_start = min(max(a.query_start_loc[r], 0), a.num_tokens);
  g.L = min(min(a.query_start_loc[r + 1] - g.q_start, a.max_query_len), a.num_tokens - g.q_start);
  g.ks = min(a.key_start[r], a.total_keys);
  g.S = min(a.key_start[r + 1], a.total_keys) - g.ks;
  return g;
}
// keys visible to some query of the tile starting at query q0 (causal,
// bottom-right aligned: query i sees keys 0 .. S - L + i)
__device__ __forceinline__ int visible_keys(const ReqGeom& g, int q0) {
  return min(g.S, max(0, g.S - g.L + min(q0 + kBM, g.L)));
}

// ------------------------------------------------------------- schedule
constexpr int kSortBuckets = 1024;

__global__ __launch_bounds__(256) void mla_schedule_kernel(MlaPrefill a) {
  __shared__ int s_sum[4];
  __shared__ int s_hist[kSortBuckets];
  __shared__ int s_max;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // key offsets: inclusive block scan of the (clamped) sequence lengths
  const int cap = a.max_blocks * a.block_size;
  int carry = 0;
  if (tid == 0) {
    a.key_start[0] = 0;
    s_max = 0;
  }
  for (int base = 0; base < a.num_seqs; base += 256) {
    const int r = base + tid;
    int v = r < a.num_seqs ? min(max(a.seq_lens[r], 0), cap) : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) s_sum[w] = v;
    __syncthreads();
    int before = carry;
    for (int i = 0; i < w; ++i) before += s_sum[i];
    if (r < a.num_seqs) a.key_start[r + 1] = before + v;
    carry += s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
    __syncthreads();
  }
  for (int i = tid; i < kSortBuckets; i += 256) s_hist[i] = 0;
  __syncthreads();   // also orders the key offsets above before the reads below

  // Requests longest first, each request's q tiles together (last, longest,
  // first): the sort key of a request is 1 + the 64-key tiles its last q tile
  // visits, coarsened by a shift so that the largest fits the buckets; bucket
  // 0 holds the longest.  Keeping a request's tiles together keeps its
  // expanded keys and values in L2 while they run.
  for (int r = tid; r < a.num_seqs; r += 256) {
    const ReqGeom g = request_geometry(a, r);
    if (g.L > 0) atomicMax(&s_max, 1 + (max(g.S, 0) + kBN - 1) / kBN);
  }
  __syncthreads();
  int shift = 0;
  while ((s_max >> shift) >= kSortBuckets) ++shift;
  auto bucket = [&](const ReqGeom& g) {
    const int cost = 1 + (max(g.S, 0) + kBN - 1) / kBN;
    return kSortBuckets - 1 - min(cost >> shift, kSortBuckets - 1);
  };
  auto q_tiles = [&](const ReqGeom& g) { return g.L > 0 ? (g.L + kBM - 1) / kBM : 0; };
  for (int r = tid; r < a.num_seqs; r += 256) {
    const ReqGeom g = request_geometry(a, r);
    const int nq = q_tiles(g);
    if (nq > 0) atomicAdd(&s_hist[bucket(g)], nq);
  }
  __syncthreads();
  // exclusive scan of the histogram (in items): 4 buckets per thread
  int loc[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    loc[i] = sum;
    sum += s_hist[4 * tid + i];
  }
  int v = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  __syncthreads();
  if (lane == 63) s_sum[w] = v;
  __syncthreads();
  int before = v - sum;
  for (int i = 0; i < w; ++i) before += s_sum[i];
  const int n_items = s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) s_hist[4 * tid + i] = before + loc[i];
  __syncthreads();
  // placement (the order of requests within a bucket is arbitrary: each
  // item's result does not depend on where it runs)
  for (int r = tid; r < a.num_seqs; r += 256) {
    const ReqGeom g = request_geometry(a, r);
    const int nq = q_tiles(g);
    if (nq == 0) continue;
    const int pos = atomicAdd(&s_hist[bucket(g)], nq);
    for (int i = 0; i < nq && pos + i < a.item_cap; ++i)
      reinterpret_cast<int2*>(a.items)[pos + i] = make_int2(r, nq - 1 - i);
  }
  if (tid == 0) *a.n_items = min(n_items, a.item_cap);
}

// ------------------------------------------------------------- attention kernel
__global__ __launch_bounds__(256, 2) void mla_attn_kernel(MlaPrefill a) {
  __shared__ __align__(16) char smem[2 * kAStage];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int H = a.num_heads;
  // work-group -> (item of the work list, head): items longest first, the
  // heads of an item consecutive (with H a multiple of 8, head h of every
  // item runs on XCD h % 8, where its expanded rows stay in L2)
  const int id = blockIdx.x;
  const int item = id / H, h = id % H;
  if (item >= *a.n_items) return;
  const int2 it = reinterpret_cast<const int2*>(a.items)[item];
  const int r = it.x, qt = it.y;
  const ReqGeom geom = request_geometry(a, r);
  const int q_start = geom.q_start, L = geom.L, ks = geom.ks, S = geom.S;
  const int q0 = qt * kBM;
  if (q0 >= L || L <= 0) return;
  const int C = S - L;
  const int kv_end = visible_keys(geom, q0);
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // ---- Q fragments: nope dims 16 kk + 8 (l / 32), rope dims likewise
  const int my_row = q0 + wave * 32 + (lane & 31);
  const bool row_ok = my_row < L;
  u32x4_t qf[8], qr[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         int64_t(q_start + (row_ok ? my_row : 0)) * a.q_st + int64_t(h) * a.q_sh +
                         8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = row_ok ? load16(qp + 16 * kk) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qr[kk] = row_ok ? load16(qp + kDn + 16 * kk) : u32x4_t{0, 0, 0, 0};
  }

  // ---- gather of one tile (keys of the request are contiguous rows)
  const char* kbase = static_cast<const char*>(a.k_exp) + (int64_t(ks) * H + h) * (kDq * 2);
  const char* vbase = static_cast<const char*>(a.v_exp) + (int64_t(ks) * H + h) * (kDv * 2);
  const int64_t kstride = int64_t(H) * kDq * 2, vstride = int64_t(H) * kDv * 2;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // Lane offsets of the DMA loads within a tile of 64 keys: nope and value
  // rows (4 rows x 256 B per load, wave w: loads w + 4 jj), rope rows (8 rows
  // x 128 B).  A full tile adds only a scalar base; the last tile clamps rows
  // past its end to the last visible key.
  uint32_t koff[4], voff[4], poff[2];
  int krow[4], prow[2];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int row = 4 * (wave + 4 * jj) + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    krow[jj] = row;
    koff[jj] = uint32_t(row * kstride + 16 * c);
    voff[jj] = uint32_t(row * vstride + 16 * c);
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int row = 8 * (wave + 4 * jj) + (lane >> 3);
    prow[jj] = row;
    poff[jj] = uint32_t(row * kstride + kNRow + 16 * pslot(row, lane & 7));
  }
  auto gload = [&](int tile, char* dst) {
    char* dk = dst;
    char* dv = dst + kNTile;
    char* dp = dst + 2 * kNTile;
    const int key0 = tile * kBN;
    const char* kb = kbase + int64_t(key0) * kstride;
    const char* vb = vbase + int64_t(key0) * vstride;
    if (key0 + kBN <= kv_end) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = wave + 4 * jj;
        __builtin_amdgcn_global_load_lds(kb + koff[jj], (lds_ptr)(dk + 1024 * j), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + voff[jj], (lds_ptr)(dv + 1024 * j), 16, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        __builtin_amdgcn_global_load_lds(kb + poff[jj], (lds_ptr)(dp + 1024 * (wave + 4 * jj)), 16, 0, 0);
    } else {
      const int last = kv_end - 1 - key0;   // rows past it re-read the last visible key
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = wave + 4 * jj;
        const int back = krow[jj] - min(krow[jj], last);
        __builtin_amdgcn_global_load_lds(kb + (koff[jj] - uint32_t(back * kstride)),
                                         (lds_ptr)(dk + 1024 * j), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + (voff[jj] - uint32_t(back * vstride)),
                                         (lds_ptr)(dv + 1024 * j), 16, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int back = prow[jj] - min(prow[jj], last);
        __builtin_amdgcn_global_load_lds(kb + (poff[jj] - uint32_t(back * kstride)),
                                         (lds_ptr)(dp + 1024 * (wave + 4 * jj)), 16, 0, 0);
      }
    }
  };
  auto gwait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };

  const float scale2 = fmaxf(a.scale * kLog2e, 0x1p-126f);
  float m_run = kNoMax, l_run = 0.0f;
  f32x16_t acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;

  if (n_tiles > 0) {
    gload(0, smem);
    gwait();
  }
  __syncthreads();
  const int row_abs = C + my_row;
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1, smem + (buf ^ 1) * kAStage);
    const char* kt = smem + buf * kAStage;
    const char* vt = kt + kNTile;
    const char* pt = kt + 2 * kNTile;
    const int key0 = t * kBN;

    // S^T for two 32-key halves: 8 k-steps over the nope tile, 4 over rope
    f32x16_t s[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[hh][i] = 0.0f;
    {
      // 12 k-steps (8 over the nope tile, 4 over rope), the two 32-key halves
      // a constant offset apart; reads one step ahead of the MFMAs, issued as
      // inline assembly (see the expansion) and waited for explicitly
      // kQD k-steps of reads in flight ahead of the MFMAs (LDS latency is
      // longer than the two MFMAs of a step)
      constexpr int kQD = 2;
      const int kr = lane & 31, hi = lane >> 5;
      u32x4_t kf[kQD + 1][2];
      auto issue = [&](auto kc) {
        constexpr int kk = decltype(kc)::value, b = kk % (kQD + 1);
        if constexpr (kk < 8) {
          const char* p = kt + kr * kNRow + 16 * ((2 * kk + hi) ^ swz(kr));
          kf[b][0] = lds_read16_issue<0>(p);
          kf[b][1] = lds_read16_issue<32 * kNRow>(p);
        } else {
          const char* p = pt + kr * kPRow + 16 * pslot(kr, 2 * (kk - 8) + hi);
          kf[b][0] = lds_read16_issue<0>(p);
          kf[b][1] = lds_read16_issue<32 * kPRow>(p);
        }
      };
      // the MFMA phases run at raised wave priority: of the two work-groups
      // sharing a SIMD, the one issuing MFMAs keeps the matrix unit fed and
      // the other's softmax takes the free issue slots
      __builtin_amdgcn_s_setprio(1);
      static_for<kQD>([&](auto kc) { issue(kc); });
      static_for<12>([&](auto kc) {
        constexpr int kk = decltype(kc)::value, b = kk % (kQD + 1);
        if constexpr (kk + kQD < 12) issue(std::integral_constant<int, kk + kQD>{});
        // reads of the later steps still in flight: 2 per step
        constexpr int kLater = 2 * (kk + kQD < 12 ? kQD : 11 - kk);
        lds_wait<kLater>(kf[b][0], kf[b][1]);
        const u32x4_t& qk = kk < 8 ? qf[kk < 8 ? kk : 0] : qr[kk < 8 ? 0 : kk - 8];
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[b][0]), as_bf16x8(qk), s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[b][1]), as_bf16x8(qk), s[1], 0, 0, 0);
      });
    }

    __builtin_amdgcn_s_setprio(0);
    // online softmax (lazy rescale as in the varlen prefill kernel)
    const bool need_mask = (key0 + kBN > kv_end) || (key0 + kBN - 1 > C + q0 + wave * 32);
    u32x4_t pf[4];
    float psum = 0.0f, alpha = 1.0f;
    bool rescale = false;
    auto update = [&](auto masked_tag) {
      constexpr bool kMasked = decltype(masked_tag)::value;
      if constexpr (kMasked) {
        const int lim = min(kv_end - 1, row_abs) - key0 - 4 * (lane >> 5);
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
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    }

    // O^T += V^T P^T (transposing LDS reads of the value tile)
    const int grp = lane >> 4, gi = lane & 15, kg = lane >> 5;
    const int c0 = 2 * (grp & 1) + ((gi & 3) >> 1);
    const int vr0 = 4 * kg + (gi >> 2);
    const char* vb[2][4];   // key rows vr0 (+ 8), d-tile dt; 16 ks rows further is a constant
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vb[e][dt] = vt + (vr0 + 8 * e) * kNRow + 16 * ((4 * dt + c0) ^ swz(vr0 + 8 * e)) + 8 * (gi & 1);
    // kVD steps of transposing reads in flight ahead of the MFMAs
    constexpr int kVD = 4;
    u32x2_t vr[kVD + 1][2];
    auto vissue = [&](auto ic) {
      constexpr int i = decltype(ic)::value, ks4 = i / 4, dt = i % 4, b = i % (kVD + 1);
      vr[b][0] = lds_read_tr_issue<16 * ks4 * kNRow>(vb[0][dt]);
      vr[b][1] = lds_read_tr_issue<16 * ks4 * kNRow>(vb[1][dt]);
    };
    __builtin_amdgcn_s_setprio(1);
    static_for<kVD>([&](auto ic) { vissue(ic); });
    static_for<16>([&](auto ic) {
      constexpr int i = decltype(ic)::value, ks4 = i / 4, dt = i % 4, b = i % (kVD + 1);
      if constexpr (i + kVD < 16) vissue(std::integral_constant<int, i + kVD>{});
      constexpr int kLater = 2 * (i + kVD < 16 ? kVD : 15 - i);
      lds_wait<kLater>(vr[b][0], vr[b][1]);
      const u32x4_t vf = u32x4_t{vr[b][0].x, vr[b][0].y, vr[b][1].x, vr[b][1].y};
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks4]), acc[dt], 0, 0, 0);
    });

    __builtin_amdgcn_s_setprio(0);
    if (t + 1 < n_tiles) {
      // this wave's loads of tile t + 1 have landed; after the barrier
      // everyone's have, and everyone is done reading this tile's buffer
      gwait();
      __builtin_amdgcn_s_barrier();
    }
  }

  const float l_tot = xor32_sum(l_run);
  if (!row_ok) return;
  const int64_t orow = int64_t(q_start) + my_row;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* op = static_cast<uint16_t*>(a.out) + (orow * H + h) * kDv;
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
    a.lse[orow * H + h] = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_mla_prefill(const MlaPrefill& a, hipStream_t s) {
  if (a.num_seqs <= 0 || a.num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_schedule_kernel, dim3(1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.total_keys > 0) {
    const int64_t g_tiles = (int64_t(a.total_keys) + kEN - 1) / kEN;
    const int64_t wgs = (g_tiles + kXcds - 1) / kXcds * kXcds * (2 * int64_t(a.num_heads));
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_expand_kernel, dim3(unsigned(wgs)), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.max_query_len <= 0) return hipSuccess;
  const int64_t n_qt = (a.max_query_len + kBM - 1) / kBM;
  const int64_t items = std::min<int64_t>(int64_t(a.num_seqs) * n_qt, a.item_cap);
  const int64_t wgs = items * a.num_heads;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_attn_kernel, dim3(unsigned(wgs)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
