// MLA decode over the latent cache, split-KV partials merged by LSE.
//
// Method: "Triton 與 MLA：可移植注意力與潛空間注意力" (設計動機, 資料流): the cache
// holds one row [kv_c (512) | k_pe (64)] per token, read as a single key
// head shared by every query head (MQA); the query is [q_nope | q_pe]; the
// value is the first 512 columns of the same row; partial outputs of each KV
// split carry their lse for the stage-2 merge.  Online softmax as in
// "第 1 章 注意力后端" §4.1.
//
// gfx950 mapping.  One work-group of 4 waves (one per SIMD) walks a run of
// 32-key tiles for all H <= 128 query heads; wave w owns heads 32w..32w+31
// (heads past H compute head 0's scores; their results are dropped).  Every head
// reads the same latent row, so both products are dense contractions on
// v_mfma_f32_32x32x16_bf16, computed transposed so that each lane owns one
// head:
//   S^T[32 keys x 32 heads] = K[32 x 576] Q^T[576 x 32]   (36 k-steps)
//   O^T[512 x 32 heads]    += V^T[512 x 32] P^T[32 x 32]  (16 d-tiles x 2)
// P^T is the S^T output registers (bf16), V^T comes from gfx950's
// transposing LDS read.  With 32 heads per operand each LDS byte read feeds
// twice the MFMA work of a 16-head split, and the 256-register O^T
// accumulator lives in the AGPRs of a wave that has its SIMD to itself.
// Each latent row is fetched from HBM once per work-group into an LDS tile
// (global_load_lds_dwordx4, four buffers) and feeds both products.  The
// tiles are software-pipelined: while tile t's scores are computed, tile t - 1
// waits for its value product, which runs with tile t's softmax in its MFMA
// shadow, and tiles t + 1, t + 2 are loading.  The LDS operand reads are
// issued as inline assembly and waited for explicitly, three MFMAs ahead: the
// compiler cannot tell the DMA-filled buffers apart and would otherwise wait
// for every load in flight before reading any of them.  Per tile and
// work-group the four waves read 144 KB of K and 128 KB of V^T from LDS (each
// wave the whole tile), which with the tile's 36 KB of DMA writes makes LDS
// bandwidth, not the MFMAs, this kernel's limit.
#include "balanced.hpp"
#include "launch.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kRope = 64;
constexpr int kBN = 32;                         // keys per tile
constexpr int kWaves = 4;
constexpr int kHeadsPerWave = 32;
constexpr int kStages = 4;                      // LDS tile buffers: kStages - 1 tiles in flight
constexpr float kSlack = 8.0f;                  // lazy-rescale headroom, log2 units
constexpr int kKDepth = 3;                      // K-fragment reads in flight ahead of their MFMA
constexpr int kVDepth = 3;                      // V^T steps (two reads each) in flight ahead

// Sizes that follow from kv_lora_rank R (the latent row is R + 64 elements;
// R = 512 gives the 576-element head, R = 256 the 320-element one).
template <int R>
struct MlaDims {
  static constexpr int kRank = R;
  static constexpr int kRow = R + kRope;                   // elements per latent row
  static constexpr int kChunks = kRow * 2 / 16;            // 16-byte chunks per row
  static constexpr int kCG = kChunks / 8;                  // 8-chunk groups per row
  static constexpr int kRowBytes = kRow * 2;               // unpadded (swizzled)
  static constexpr int kTileBytes = kBN * kRowBytes;
  static constexpr int kTileLoads = kBN * kChunks / 64;    // wave-wide 16-byte loads per tile
  static constexpr int kLoadsPerWave = kTileLoads / kWaves;
  static constexpr int kKSteps = kRow / 16;                // k-steps of the score product
  static constexpr int kDTiles = R / 32;                   // d-tiles of the value product
  static_assert(kTileLoads % kWaves == 0 && kKSteps % 4 == 0 && kDTiles % 2 == 0, "tiling");
  static_assert(kStages * kTileBytes <= 160 * 1024 - 64, "LDS budget");
  static_assert(2 * kLoadsPerWave < 64, "vmcnt range");
  static_assert(kChunks % 8 == 0 && kLoadsPerWave == kCG && kBN == 8 * kWaves,
                "one row-block of the tile per wave");
};

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt not waited for)
template <int N>
constexpr int vmcnt_imm() { return (N & 15) | ((N >> 4) << 14) | 0x0F70; }

// LDS tile layout.  A tile is cut into 1 KiB blocks of 8 rows x 8 chunks
// (16-byte chunks, 128 bytes of a row): block (m, k) holds rows 8m .. 8m+7,
// chunks 8k .. 8k+7, and sits at 1024 (kCG m + k), kCG = chunk groups per
// row (9 for the 576-element row, 5 for the 320-element one).  Inside a
// block, row r takes 128 bytes at 128 (r % 8), and chunk c of it sits in slot
// (c % 8) ^ sx(r), with sx(r) holding bits 1, 2 and 3 of r in reverse order.
// Modulo the 256 bytes of one pass over the banks an address is then
// 128 (r % 2) + 16 ((c % 8) ^ sx(r)), so
// * a 16-lane phase of a K-fragment read (16 consecutive rows, one chunk)
//   hits 16 distinct 16-byte bank groups, and
// * a 32-lane phase of a V^T transposing read (4 consecutive rows 4q..4q+3,
//   4 consecutive chunks 4m..4m+3, both 8-byte halves) does the same,
// so neither read has bank conflicts.  A block is one wave-wide 16-byte DMA
// load whose lanes fetch from 8 rows of the cache: wave w fetches row-block
// w, one per-lane address per tile plus 128 k for block k.
__device__ __forceinline__ int sx(int r) {
  return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}
template <int kCG>
__device__ __forceinline__ int lds_off(int r, int c) {
  return 1024 * (kCG * (r >> 3) + (c >> 3)) + 128 * (r & 7) + 16 * ((c & 7) ^ sx(r));
}

// The two products are issued as inline assembly so that each keeps its own
// register file: the 256-register O^T accumulator in AGPRs, the score
// accumulator (read by the softmax) in VGPRs.  With the builtin the compiler
// picks one form for every MFMA of the kernel.  The hazards the compiler
// would otherwise cover are covered by explicit s_nop below (an MFMA result
// read by the VALU, a VALU result read by an MFMA).
__device__ __forceinline__ void mfma_s0(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Orders every read and write of the accumulator tiles after (tie) or
// before (hazard fence) this point; kNop wait states go after the last one.
__device__ __forceinline__ void acc_tie4(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d) {
  asm volatile("" : "+a"(a), "+a"(b), "+a"(c), "+a"(d));
}
template <int kNop, int N>
__device__ __forceinline__ void acc_fence(f32x16_t (&acc)[N]) {
  static_assert(N % 4 == 0 && N >= 4, "groups of four tiles");
#pragma unroll
  for (int g = 0; g + 4 < N; g += 4) acc_tie4(acc[g], acc[g + 1], acc[g + 2], acc[g + 3]);
  asm volatile("s_nop %4" : "+a"(acc[N - 4]), "+a"(acc[N - 3]), "+a"(acc[N - 2]), "+a"(acc[N - 1])
               : "n"(kNop));
}

// Two schedules share the kernel body:
// * kBalanced = false: work-group (request, split) over keys [t0, t1) of one
//   request, split s = [s P, (s+1) P); partials [B, H, S, 513] for the merge.
// * kBalanced = true: work-group j walks chunk range j of the batch's chunk
//   list (balanced.hpp), finishing the requests inside it and leaving segment
//   partials [(nr + B) H, 516] for the others.
// A "tile" is 32 keys [kb + 32 lc, kb + 32 lc + 32) of request r, keys at or
// past kend masked (split: kb = t0, kend = t1; balanced: kb = 0, kend = len).
// kFp8 (balanced schedule only): the cache holds E4M3 codes, one scale for
// the whole row.  A tile's 18 KiB of codes is gathered into an LDS staging
// ring (four stages, 16-byte DMA pieces: waves 0 and 1 issue five, waves 2
// and 3 four), then widened once per work-group to the bf16 tile layout
// above (v_cvt_scalef32_pk_bf16_fp8, exact) in one of two bf16 buffers, so
// both products run unchanged; the scale multiplies the score scale and the
// final normalisation.
constexpr int kF8TileBytes = kBN * (512 + kRope);        // 18432 B of codes (kv_lora_rank 512)
constexpr int kF8Pieces = kF8TileBytes / 1024;           // 18 wave-wide 16-byte loads
constexpr int kF8Stages = 4;
constexpr int kF8Chunks = kF8TileBytes / 8 / (64 * kWaves);   // 9 eight-code chunks per thread
static_assert(2 * MlaDims<512>::kTileBytes + kF8Stages * kF8TileBytes <=
                  kStages * MlaDims<512>::kTileBytes, "fp8 LDS budget");
static_assert(kF8Pieces == 18 && kF8Chunks == 9, "fp8 piece counts");

// Page ids of a tile's first and last key.
struct Pages { int32_t b0, b1; };

template <bool kBalanced, bool kFp8, int kR>
__global__ __launch_bounds__(64 * kWaves, 1) void mla_kernel(MlaDecode a) {
  static_assert(kBalanced || !kFp8, "the FP8 cache runs on the balanced schedule");
  static_assert(!kFp8 || kR == 512, "the FP8 cache is built for kv_lora_rank 512");
  using Dm = MlaDims<kR>;
  constexpr int kRank = Dm::kRank, kRow = Dm::kRow, kChunks = Dm::kChunks;
  constexpr int kRowBytes = Dm::kRowBytes, kTileBytes = Dm::kTileBytes;
  constexpr int kTileLoads = Dm::kTileLoads, kLoadsPerWave = Dm::kLoadsPerWave;
  constexpr int kKSteps = Dm::kKSteps, kDTiles = Dm::kDTiles;
  (void)kTileLoads;
  __shared__ __align__(1024) char smem[kStages * kTileBytes];
  __shared__ int s_wave_sum[2 * kWaves];
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
    if (!balanced_range<kMlaRangeOverhead>(a.seq_lens, B, cap, a.num_ranges, j, j == 0, a.cu,
                                           s_wave_sum, s_start, c0, c1, n_tiles, cur))
      return;
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
      return next_chunk<kMlaRangeOverhead>(p, a.seq_lens, cap, B);
    } else {
      return ChunkPos{p.r, p.lc + 1, p.len, p.base};
    }
  };

  const int c32 = lane & 31;          // head column / key row / dim row of the MFMA operands
  const int g = lane >> 5;            // k half of the MFMA operands
  const bool active = kHeadsPerWave * wave < H;
  const int head = kHeadsPerWave * wave + c32;
  const bool head_ok = head < H;

  // ---- Q^T fragments (B operand of S^T): head `head`, dims 16 kk + 8 g .. + 8
  u32x4_t qf[kKSteps];
  auto load_q = [&](int r) {
    const int hq = head_ok ? head : 0;
    const uint16_t* qn = static_cast<const uint16_t*>(a.q_nope) + int64_t(r) * a.qn_sb +
                         int64_t(hq) * a.qn_sh + 8 * g;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_pe) + int64_t(r) * a.qp_sb +
                         int64_t(hq) * a.qp_sh + 8 * g;
    // heads past H read head 0 (in bounds) and are zeroed after the wait
#pragma unroll
    for (int kk = 0; kk < kRank / 16; ++kk) qf[kk] = load16(qn + 16 * kk);
#pragma unroll
    for (int kk = 0; kk < kRope / 16; ++kk) qf[kRank / 16 + kk] = load16(qp + 16 * kk);
  };

  // ---- gather of a tile straight into LDS (global_load_lds_dwordx4; lane i
  // lands at byte 16 i of the load's 1 KiB): wave w fetches row-block w, lane
  // i row 8 w + i / 8, slot i % 8 of each of the row's kCG blocks.  The lane's
  // source is one address per tile: its row on page b0 or b1, the chunk of
  // its slot; block k adds 128 k.  Rows at or past kend re-read key kend - 1
  // (finite, masked out below).
  const char* cache = static_cast<const char*>(a.cache);
  const int my_row = 8 * wave + (lane >> 3);
  const int lane_sw = 16 * ((lane & 7) ^ sx(my_row));
  // Page ids of a tile's first and last key (scalar loads).  They are read a
  // step before the gather that uses them, at the end of the previous tile's
  // compute: a scalar load waited for right before its use would stall the
  // gather's issue, and one in flight during the LDS operand reads would
  // stall those (both count on lgkmcnt).
  auto pages = [&](const ChunkPos& p) {
    const int32_t* table = a.block_table + int64_t(p.r) * a.max_blocks;
    const int key0 = kb + p.lc * kBN;
    const int kend = p.len;
    const int kl0 = min(key0, kend - 1), kl1 = min(key0 + kBN - 1, kend - 1);
    return Pages{uniform_load(table + kl0 / bs), uniform_load(table + kl1 / bs)};
  };
  auto gsrc = [&](const ChunkPos& p, const Pages& pg) __attribute__((always_inline)) {
    const int key0 = kb + p.lc * kBN;
    int64_t b0 = pg.b0, b1 = pg.b1;
    b0 = (b0 < 0 || b0 >= a.num_blocks) ? 0 : b0;
    b1 = (b1 < 0 || b1 >= a.num_blocks) ? 0 : b1;
    const int in0 = key0 - (key0 / bs) * bs;        // key0's row within page b0
    const int ip = in0 + min(my_row, p.len - 1 - key0);   // row within page b0, may run past it
    const int64_t row = ip < bs ? b0 * bs + ip : b1 * bs + (ip - bs);
    return cache + row * kRowBytes + lane_sw;
  };
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // block k of the tile in buffer `stage`; cache policy 2 = non-temporal:
  // every latent row is read once
  auto gissue = [&](const char* src, int stage, int k) __attribute__((always_inline)) {
    __builtin_amdgcn_global_load_lds(src + 128 * k,
                                     (lds_ptr)(smem + stage * kTileBytes + 1024 * (Dm::kCG * wave + k)),
                                     16, 0, 2);
  };
  auto gload = [&](const ChunkPos& p, int stage, const Pages& pg) __attribute__((always_inline)) {
    const char* src = gsrc(p, pg);
#pragma unroll
    for (int k = 0; k < kLoadsPerWave; ++k) gissue(src, stage, k);
  };
  auto gwait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  // ---- FP8: gather of a tile's codes into staging stage `stage` (the tile's
  // rows contiguous, 576 B each), pieces I = wave + 4 jj < 18, lane l at
  // byte 1024 I + 16 l; the same page / kend correction as the bf16 gather.
  constexpr int kF8Row = kRow;   // bytes of codes per row
  const int f8_n = wave < 2 ? 5 : 4;   // pieces this wave issues per tile
  auto gload8 = [&](const ChunkPos& p, int stage, const Pages& pg) {
    const int key0 = kb + p.lc * kBN;
    const int kend = p.len;
    int64_t b0 = pg.b0, b1 = pg.b1;
    b0 = (b0 < 0 || b0 >= a.num_blocks) ? 0 : b0;
    b1 = (b1 < 0 || b1 >= a.num_blocks) ? 0 : b1;
    const int in0 = key0 - (key0 / bs) * bs;
    const char* c8 = static_cast<const char*>(a.cache);
    const char* base0 = c8 + (b0 * bs + in0) * int64_t(kF8Row);
    const char* base1 = c8 + (b1 * bs - (bs - in0)) * int64_t(kF8Row);
    const bool simple = in0 + kBN <= bs && key0 + kBN <= kend;   // wave-uniform
    const int last = kend - 1 - key0;
    typedef __attribute__((address_space(3))) void* lds_ptr;
    char* dst = smem + 2 * kTileBytes + stage * kF8TileBytes;
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      if (jj == 4 && wave >= 2) break;
      const uint32_t off = uint32_t(1024 * (wave + kWaves * jj) + 16 * lane);
      const char* src = base0 + off;
      if (!simple) {
        const int row = int(off / uint32_t(kF8Row));
        const int rr = min(row, last);
        src = (in0 + rr < bs ? base0 : base1) + int64_t(off) + int64_t(rr - row) * kF8Row;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_ptr)(dst + 1024 * (wave + kWaves * jj)), 16, 0, 2);
    }
  };
  // tile t's codes have landed for this wave when at most f8_n x (tiles
  // issued after t) of its loads are outstanding
  auto wait_tiles8 = [&](int k) {
    if (k <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
    else if (k == 1) {
      if (f8_n == 5) __builtin_amdgcn_s_waitcnt(0x0F75);             // vmcnt(5)
      else __builtin_amdgcn_s_waitcnt(0x0F74);                       // vmcnt(4)
    } else if (k == 2) {
      if (f8_n == 5) __builtin_amdgcn_s_waitcnt(0x0F7A);             // vmcnt(10)
      else __builtin_amdgcn_s_waitcnt(0x0F78);                       // vmcnt(8)
    } else {
      if (f8_n == 5) __builtin_amdgcn_s_waitcnt(0x0F7F);             // vmcnt(15)
      else __builtin_amdgcn_s_waitcnt(0x4F70);                       // vmcnt(16)
    }
  };
  // staging `stage` -> bf16 buffer `buf`: thread chunk pos = tid + 256 i is
  // row pos / 72, chunk pos % 72 (codes 8 c .. 8 c + 7), written to its
  // swizzled slot.  The LDS accesses are inline assembly so that they stay
  // ordered against the bare barriers around them.
  auto convert8 = [&](int stage, int buf) {
    const uint32_t src = lds_addr(smem) + uint32_t(2 * kTileBytes + stage * kF8TileBytes + 8 * tid);
    const uint32_t dst = lds_addr(smem) + uint32_t(buf * kTileBytes);
    u32x2_t c[kF8Chunks];
    static_for<kF8Chunks>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      c[i] = lds_read8_at<2048 * i>(src);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]),
                 "+v"(c[4]), "+v"(c[5]), "+v"(c[6]), "+v"(c[7]), "+v"(c[8]));
#pragma unroll
    for (int i = 0; i < kF8Chunks; ++i) {
      const int pos = tid + 256 * i;
      const int row = pos / kChunks;
      const int ch = pos - row * kChunks;
      const u32x4_t w = u32x4_t{fp8x2_to_bf16x2<false>(c[i].x), fp8x2_to_bf16x2<true>(c[i].x),
                                fp8x2_to_bf16x2<false>(c[i].y), fp8x2_to_bf16x2<true>(c[i].y)};
      const uint32_t addr = dst + uint32_t(lds_off<Dm::kCG>(row, ch));
      lds_write16_at(addr, w);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // ---- LDS operand addresses (per lane; the stage and the k-step / d-tile
  // group are added as offsets)
  // K fragment of k-step kk = 4 q + kq: key row c32, chunk 8 q + 2 kq + g.
  const uint32_t lds0 = lds_addr(smem);
  uint32_t kaddr[4];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq)
    kaddr[kq] = lds0 + lds_off<Dm::kCG>(c32, 2 * kq + g);
  // V^T fragment of d-tile m = 2 mh + ml and key step st, read e (0, 1):
  // within each 16-lane group, lane 4 q + i reads key row 16 st + 8 e + 4 g
  // + q, dims 32 m + 16 (lane / 16 % 2) + 4 i .. + 4 (chunk 4 m + c0, half
  // i % 2, c0 = 2 (lane / 16 % 2) + i / 2); the transposing read hands lane
  // 4 q + i of the group dim 16 (lane / 16 % 2) + 4 q + i, keys +0..3, which
  // is the A layout of v_mfma_f32_32x32x16_bf16 for keys in the order of the
  // S^T output registers.
  uint32_t vaddr[2][2];   // [e][ml]
  {
    const int i4 = lane & 3, q4 = (lane >> 2) & 3;
    const int cg = 2 * ((lane >> 4) & 1) + (i4 >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 8 * e + 4 * g + q4;
#pragma unroll
      for (int ml = 0; ml < 2; ++ml)
        vaddr[e][ml] = lds0 + lds_off<Dm::kCG>(row, 4 * ml + cg) + 8 * (i4 & 1);
    }
  }

  // Masked scores are -inf and meet the scale inside the exponent; a zero
  // scale is raised to the smallest normal float so that -inf * scale stays
  // -inf (weight 0) while every visible score still maps to exp2(0) = 1.
  const float scale2 = fmaxf((kFp8 ? a.scale * a.kv_scale : a.scale) * kLog2e, 0x1p-126f);
  float m_run = kNoMax;
  float l_run = 0.0f;          // this lane's share of head `head`'s sum
  f32x16_t acc[kDTiles];       // O^T: d = 32 m + 8 (r / 4) + 4 g + r % 4
#pragma unroll
  for (int m = 0; m < kDTiles; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;

  // ---- finish a segment: per-head sum over lanes l, l ^ 32, normalise, write
  auto finish = [&](const ChunkPos& p) {
    acc_fence<15>(acc);   // the VALU reads the accumulator
    const float l_tot = xor32_sum(l_run);
    if (!active || !head_ok) return;
    const float inv = (kFp8 ? a.kv_scale : 1.0f) / l_tot;
    const float lse_nat = (m_run + fast_log2(l_tot)) * kLn2;
    const int64_t row = int64_t(p.r) * H + head;
    bool direct;
    float* pp;
    int pstride;   // floats per partial row
    if constexpr (kBalanced) {
      direct = p.base >= c0 && p.base + chunks_of(p.len) <= c1;
      pp = a.part + (int64_t(j + p.r) * H + head) * (kRank + 4);
      pstride = kRank + 4;
    } else {
      direct = a.direct;
      pp = a.part + (row * a.num_splits + s) * (kRank + 1);
      pstride = kRank + 1;
    }
    // one accumulator tile at a time through the VGPRs
    if (direct) {
      uint16_t* op = static_cast<uint16_t*>(a.out) + row * kRank;
#pragma unroll
      for (int m = 0; m < kDTiles; ++m) {
        asm volatile("" : "+a"(acc[m]));
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 w;
          w.x = pack_bf16x2(acc[m][4 * q4 + 0] * inv, acc[m][4 * q4 + 1] * inv);
          w.y = pack_bf16x2(acc[m][4 * q4 + 2] * inv, acc[m][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(op + 32 * m + 8 * q4 + 4 * g) = w;
        }
      }
      if (g == 0 && a.lse) a.lse[row] = lse_nat;
    } else {
      if (kBalanced) {   // 16-byte aligned rows
#pragma unroll
        for (int m = 0; m < kDTiles; ++m) {
          asm volatile("" : "+a"(acc[m]));
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4_t*>(pp + 32 * m + 8 * q4 + 4 * g) =
                f32x4_t{acc[m][4 * q4] * inv, acc[m][4 * q4 + 1] * inv, acc[m][4 * q4 + 2] * inv,
                        acc[m][4 * q4 + 3] * inv};
        }
      } else {
#pragma unroll
        for (int m = 0; m < kDTiles; ++m) {
          asm volatile("" : "+a"(acc[m]));
#pragma unroll
          for (int i = 0; i < 16; ++i) pp[32 * m + 8 * (i >> 2) + 4 * g + (i & 3)] = acc[m][i] * inv;
        }
      }
      if (g == 0) pp[kRank] = lse_nat;
    }
    (void)pstride;
  };

  // Tile pipeline (bf16): while tile t's scores and tile t - 1's values are
  // computed, kStages - 2 tiles are loading.  Each wave issues 9 of a tile's
  // 36 loads, so "tile t has landed" is "at most 9 x (tiles issued after t)
  // loads outstanding".
  auto wait_tiles = [&](int k) {   // k = tiles issued after the one waited for
    if (k <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);                               // vmcnt(0)
    else if (k == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm<Dm::kLoadsPerWave>());
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * Dm::kLoadsPerWave>());
  };
  static_assert(kStages <= 4, "wait_tiles counts");

  auto zero_pad_q = [&]() {
    if (!head_ok) {
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qf[kk] = u32x4_t{0, 0, 0, 0};
    }
  };
  load_q(cur.r);
  gwait();   // q is in registers before any tile load is issued
  zero_pad_q();
  ChunkPos ld = cur;   // next tile to load
  int n_loaded = 0;
  constexpr int kAhead = kFp8 ? kF8Stages - 1 : kStages - 2;   // tiles loaded ahead
  for (; n_loaded < kAhead && n_loaded < n_tiles; ++n_loaded) {
    if constexpr (kFp8) gload8(ld, n_loaded, pages(ld));
    else gload(ld, n_loaded, pages(ld));
    if (n_loaded + 1 < n_tiles) ld = advance(ld);
  }
  Pages pg_next = pages(ld);   // ld stays inside the run, so this read is in bounds

  // O^T += V^T P^T over the tile at LDS offset `off`: step n = 16 st + m
  // (d-tile m, key step st), two transposing reads per step, issued kVDepth
  // steps ahead; between(n) runs right after step n's MFMA
  auto pv = [&](const u32x4_t (&pfx)[2], uint32_t off, auto&& between) __attribute__((always_inline)) {
    uint32_t vb[2][2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int ml = 0; ml < 2; ++ml) vb[e][ml] = vaddr[e][ml] + off;
    constexpr int kD = kVDepth;
    u32x2_t vr[kD + 1][2];
    auto vissue = [&](auto nc) __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value, st = n / kDTiles, m = n % kDTiles;
      constexpr int o = 2048 * Dm::kCG * st + 1024 * (m / 2);   // row-blocks 2 st.., block m / 2
      vr[n % (kD + 1)][0] = lds_read_tr_at<o>(vb[0][m % 2]);
      vr[n % (kD + 1)][1] = lds_read_tr_at<o>(vb[1][m % 2]);
    };
    static_for<kD>([&](auto nc) __attribute__((always_inline)) { vissue(nc); });
    static_for<2 * kDTiles>([&](auto nc) __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value, st = n / kDTiles, m = n % kDTiles;
      constexpr int kN = 2 * kDTiles;
      constexpr int kLeft = 2 * (n + kD < kN ? kD : kN - 1 - n);
      if constexpr (n + kD < kN) vissue(std::integral_constant<int, n + kD>{});
      lds_wait<kLeft>(vr[n % (kD + 1)][0], vr[n % (kD + 1)][1]);
      const u32x4_t vf = u32x4_t{vr[n % (kD + 1)][0].x, vr[n % (kD + 1)][0].y,
                                 vr[n % (kD + 1)][1].x, vr[n % (kD + 1)][1].y};
      mfma_o(acc[m], vf, pfx[st]);
      between(nc);
    });
  };
  bool pend = false;           // the previous tile's value product is still to do,
  u32x4_t pf_prev[2] = {};     // with this P^T
  uint32_t prev_off = 0;       // over this LDS buffer

  // Segments: the tiles of one request within this work-group's run.  The
  // segment boundary work (write the segment, reset, load the next q) sits
  // outside the tile loop.
  int t = 0;
  for (;;) {
  const int seg_end = min(n_tiles, t + chunks_of(cur.len) - cur.lc);
  for (; t < seg_end; ++t) {
    if constexpr (kFp8) wait_tiles8(n_loaded - 1 - t);
    else wait_tiles(n_loaded - 1 - t);   // this wave's loads of tile t have landed
    // Everyone's have, and everyone is done with tile t - 1 (its LDS reads were
    // waited for).  A bare barrier: __syncthreads() would also wait for the
    // loads of the tiles still in flight.
    __builtin_amdgcn_s_barrier();
    // Refill the buffer of tile t - 1.  The bf16 tile's loads are spread
    // through the score MFMAs below (one every four k-steps): issued back to
    // back they would hold the wave for the ~16 cycles per load that the CU's
    // address unit takes.
    bool refill = false;
    const char* rsrc = cache;
    int rstage = 0;
    if (n_loaded < n_tiles) {
      if constexpr (kFp8) {
        gload8(ld, n_loaded % kF8Stages, pg_next);
      } else {
        rsrc = gsrc(ld, pg_next);
        rstage = n_loaded % kStages;
        refill = true;
        if (!active) gload(ld, rstage, pg_next);   // no MFMAs to spread them over
      }
      if (++n_loaded < n_tiles) ld = advance(ld);
    }
    if constexpr (kFp8) {
      // widen tile t into bf16 buffer t % 2 (last read by tile t - 2, which
      // every wave finished before the previous barrier); then everyone's
      // part is in place
      convert8(t % kF8Stages, t & 1);
      __builtin_amdgcn_s_barrier();
    }
    const uint32_t st_off = uint32_t((kFp8 ? (t & 1) : (t % kStages)) * kTileBytes);
    const int key0 = kb + cur.lc * kBN;
    const int kend = cur.len;
    if (active) {
      // S^T: keys 8 (i / 4) + 4 g + i % 4 (register i), head c32.  K reads
      // run kKDepth k-steps ahead.
      f32x16_t sc;
      {
        uint32_t kb4[4];
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) kb4[kq] = kaddr[kq] + st_off;
        constexpr int kD = kKDepth;
        u32x4_t kr[kD + 1];
        auto issue = [&](auto kc) __attribute__((always_inline)) {
          constexpr int kk = decltype(kc)::value;
          kr[kk % (kD + 1)] = lds_read16_at<1024 * (kk / 4)>(kb4[kk % 4]);   // block kk / 4
        };
        static_for<kD>([&](auto kc) __attribute__((always_inline)) { issue(kc); });
        static_for<kKSteps>([&](auto kc) __attribute__((always_inline)) {
          constexpr int kk = decltype(kc)::value;
          // reads of k-steps kk + 1 .. kk + kD may stay in flight
          constexpr int kLeft = kk + kD < kKSteps ? kD : kKSteps - 1 - kk;
          if constexpr (kk + kD < kKSteps) issue(std::integral_constant<int, kk + kD>{});
          lds_wait1<kLeft>(kr[kk % (kD + 1)]);
          if constexpr (kk == 0) mfma_s0(sc, kr[0], qf[0]);
          else mfma_s(sc, kr[kk % (kD + 1)], qf[kk]);
          if constexpr (!kFp8 && kk % 4 == 2 && kk / 4 < kLoadsPerWave) {
            if (refill) gissue(rsrc, rstage, kk / 4);
          }
        });
        // the VALU reads the scores: 16 wait states after the last MFMA
        asm volatile("s_nop 15" : "+v"(sc));
      }

      // Online softmax of tile t in pieces, piece n placed after MFMA n of
      // the previous tile's value product (when there is one), so that it
      // runs in the MFMAs' shadow; the empty asm statements hold each piece
      // between its neighbours.  Lazy rescale: the reference max only moves
      // when a head's max grows by more than kSlack (log2 units), so
      // p <= 2^kSlack in between; the accumulator itself is rescaled after
      // that product.
      float tmax = -INFINITY, m_new = m_run, alpha = 1.0f, psum = 0.0f;
      bool need = false;
      float pr[16];
      u32x4_t pf[2];
      auto sm = [&](auto nc) __attribute__((always_inline)) {
        constexpr int n = decltype(nc)::value;
        if constexpr (n == 0) {
          if (key0 + kBN > kend) {   // tail tile: keys at or past kend weigh 0
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (key0 + 8 * (i >> 2) + 4 * g + (i & 3) >= kend) sc[i] = -INFINITY;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) tmax = fmaxf(tmax, sc[i]);
          asm volatile("" : "+v"(tmax));
        } else if constexpr (n == 1) {
#pragma unroll
          for (int i = 8; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
          tmax = xor32_max(tmax);
          const float tm = tmax == -INFINITY ? -INFINITY : tmax * scale2;
          need = __any(tm > m_run + kSlack);
          m_new = need ? fmaxf(m_run, tm) : m_run;
          asm volatile("" : "+v"(m_new));
        } else if constexpr (n == 2) {
          alpha = fast_exp2(m_run - m_new);
          asm volatile("" : "+v"(alpha));
        } else if constexpr (n >= 3 && n < 19) {
          constexpr int i = n - 3;
          float x = sc[i];
          asm volatile("" : "+v"(x));
          pr[i] = fast_exp2(fmaf(x, scale2, -m_new));
          psum += pr[i];
          asm volatile("" : "+v"(pr[i]), "+v"(psum));
        } else if constexpr (n >= 19 && n < 23) {
          constexpr int w = 2 * (n - 19);   // words w, w + 1 of the 8 of P^T
          uint32_t lo = pack_bf16x2(pr[2 * w], pr[2 * w + 1]);
          uint32_t hi = pack_bf16x2(pr[2 * w + 2], pr[2 * w + 3]);
          asm volatile("" : "+v"(lo), "+v"(hi));
          pf[w / 4][w % 4] = lo;
          pf[w / 4][w % 4 + 1] = hi;
        } else if constexpr (n == 23) {
          l_run = l_run * alpha + psum;
          m_run = m_new;
          asm volatile("" : "+v"(l_run), "+v"(m_run));
        }
      };
      constexpr int kSmPieces = 24;
      if (pend) {
        // O^T += V^T P^T of tile t - 1, softmax of tile t in its shadow:
        // pieces [n P / N, (n + 1) P / N) after MFMA n of N
        pv(pf_prev, prev_off, [&](auto nc) __attribute__((always_inline)) {
          constexpr int kN = 2 * kDTiles, n = decltype(nc)::value;
          constexpr int lo = n * kSmPieces / kN, hi = (n + 1) * kSmPieces / kN;
          static_for<hi - lo>([&](auto jc) __attribute__((always_inline)) {
            sm(std::integral_constant<int, lo + decltype(jc)::value>{});
          });
        });
        if (need) {   // rescale the accumulator, one tile at a time through the VGPRs
          acc_fence<15>(acc);   // the value product's last results are in
#pragma unroll
          for (int m = 0; m < kDTiles; ++m) {
            asm volatile("" : "+a"(acc[m]));
            acc[m] *= alpha;
            asm volatile("" : "+a"(acc[m]));
          }
          acc_fence<4>(acc);   // written by the VALU, read by the next MFMAs
        }
      } else {
        static_for<kSmPieces>([&](auto nc) __attribute__((always_inline)) { sm(nc); });
      }
      pf_prev[0] = pf[0];
      pf_prev[1] = pf[1];
      prev_off = st_off;
      pend = true;
    }  // active
    if (n_loaded < n_tiles) pg_next = pages(ld);   // lands over the loop tail and the barrier

    if (t + 1 < seg_end) ++cur.lc;
  }
  if (pend) {   // the segment's last value product
    asm volatile("s_nop 4" : "+v"(pf_prev[0]), "+v"(pf_prev[1]));   // P^T written by the VALU
    pv(pf_prev, prev_off, [](auto) {});
    pend = false;
  }
  if (t >= n_tiles) break;
  // end of this request's keys in the run (balanced schedule only: a split
  // covers one request): emit its segment, start the next
  finish(cur);
#pragma unroll
  for (int m = 0; m < kDTiles; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;
  m_run = kNoMax;
  l_run = 0.0f;
  cur = advance(cur);
  load_q(cur.r);
  gwait();   // q (and every tile load so far) has landed
  zero_pad_q();
  }
  finish(cur);
}

}  // namespace

hipError_t launch_mla_decode(const MlaDecode& a, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  if ((a.rank != 512 && a.rank != 256) || a.rope != kRope || a.num_heads % 16 ||
      a.num_heads > kHeadsPerWave * kWaves)
    return hipErrorNotSupported;
  if (a.fp8) {
    if (a.num_ranges <= 0 || a.rank != 512) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mla_kernel<true, true, 512>), dim3(unsigned(a.num_ranges)), dim3(64 * kWaves),
                       0, s, a);
    return hipGetLastError();
  }
  if (a.num_ranges > 0) {
    if (a.rank == 512) {
      hipLaunchKernelGGL((mla_kernel<true, false, 512>), dim3(unsigned(a.num_ranges)),
                         dim3(64 * kWaves), 0, s, a);
    } else {
      hipLaunchKernelGGL((mla_kernel<true, false, 256>), dim3(unsigned(a.num_ranges)),
                         dim3(64 * kWaves), 0, s, a);
    }
    return hipGetLastError();
  }
  const int64_t wgs = int64_t(a.num_seqs) * a.num_splits;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  if (a.rank == 512) {
    hipLaunchKernelGGL((mla_kernel<false, false, 512>), dim3(unsigned(wgs)), dim3(64 * kWaves), 0, s, a);
  } else {
    hipLaunchKernelGGL((mla_kernel<false, false, 256>), dim3(unsigned(wgs)), dim3(64 * kWaves), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
