// Device-side helpers shared by the gfx950 kernels: bf16 packing, base-2
// exponentials, wave64 DPP reductions and 16-byte memory access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no key seen yet": exp2(x - kNoMax) never produces NaN.
constexpr float kNoMax = -1.0e30f;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to
// nearest even in the default rounding mode; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------- arithmetic
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Two bf16 products accumulated in fp32: a.lo*b.lo + a.hi*b.hi + c.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ----------------------------------------------------------- DPP exchange
// dpp_ctrl encodings (GCN/CDNA): quad_perm selectors, row mirror, half mirror.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140; // lane i <-> 15 - i within a row of 16
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7 - i within each 8

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}

// Sum / max over each row of 16 lanes; every lane of the row gets the result.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

// Exchange with lane ^ 16 / ^ 32 (crosses DPP rows; routed through the LDS
// crossbar by ds_bpermute, no LDS allocation).
__device__ __forceinline__ float lane_xor(float x, int m) {
  int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
      (lane ^ m) << 2, __builtin_bit_cast(int, x)));
}

// Index of the calling wave in its work-group, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// ------------------------------------------------------- scalar metadata
// Wave-uniform reads of read-only metadata (block tables, lengths) through the
// constant address space, so that they become scalar loads: those complete on
// their own counter and never make the vector-memory waits of the K/V stream
// conservative.
template <typename T>
__device__ __forceinline__ T uniform_load(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<uintptr_t>(p));
}

// ------------------------------------------------------ MFMA operand views
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Four b16 values from LDS, transposed within each 16-lane group: lane i of
// the group receives element (i % 4) of the 8-byte chunks addressed by lanes
// 4q + i/4, q = 0..3 (so a group reading a 4-row x 16-column block gets one
// column of 4 rows per lane).  ds_read_b64_tr_b16.
__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s4;
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Eight bytes from LDS, transposed within each 16-lane group: the group's
// 16 chunks of 8 bytes form 8 rows of 16 bytes (row k = the chunks of lanes
// 2k and 2k + 1), and lane i receives byte i of every row, row k in byte k.
// ds_read_b64_tr_b8.
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
__device__ __forceinline__ u32x2_t lds_read_tr8(const char* p) {
  typedef __attribute__((ext_vector_type(2))) int s32x2_t;
  typedef __attribute__((address_space(3))) s32x2_t lds_s2;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_s2*)(p)));
}

// Transposed LDS read issued as inline assembly, for tiles that are filled by
// global_load_lds: the compiler cannot tell that the read does not alias the
// tile still being filled and would wait for every outstanding load before the
// intrinsic form.  The result is NOT ready when this returns: it must pass
// through lds_wait() (which ties the registers to an s_waitcnt) before use.
template <int kOffset>
__device__ __forceinline__ u32x2_t lds_read_tr_issue(const char* p) {
  u32x2_t v;
  typedef const __attribute__((address_space(3))) char lds_char;
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)(p)));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(kOffset));
  return v;
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef const __attribute__((address_space(3))) char lds_char;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)(p)));
}
// The two reads below from a precomputed LDS byte address.
template <int kOffset>
__device__ __forceinline__ u32x2_t lds_read_tr_at(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(kOffset));
  return v;
}
template <int kOffset>
__device__ __forceinline__ u32x4_t lds_read16_at(uint32_t addr) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(kOffset));
  return v;
}

template <int kOffset>
__device__ __forceinline__ u32x2_t lds_read8_at(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(kOffset));
  return v;
}
__device__ __forceinline__ void lds_write16_at(uint32_t addr, u32x4_t v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// 16-byte LDS read issued as inline assembly (same contract as
// lds_read_tr_issue: pass the result through lds_wait() before use).
template <int kOffset>
__device__ __forceinline__ u32x4_t lds_read16_issue(const char* p) {
  u32x4_t v;
  typedef const __attribute__((address_space(3))) char lds_char;
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)(p)));
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(kOffset));
  return v;
}

// Wait until at most kLeft LDS (and scalar-memory) operations are outstanding;
// the listed registers are only read after the wait.  LDS operations complete
// in order, so the reads issued before the last kLeft ones have landed.
template <int kLeft>
__device__ __forceinline__ void lds_wait(u32x2_t& a, u32x2_t& b, u32x2_t& c, u32x2_t& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(kLeft));
}
template <int kLeft>
__device__ __forceinline__ void lds_wait(u32x2_t& a, u32x2_t& b, u32x2_t& c, u32x2_t& d,
                                         u32x2_t& e, u32x2_t& f, u32x2_t& g, u32x2_t& h) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
               : "n"(kLeft));
}

template <int kLeft>
__device__ __forceinline__ void lds_wait1(u32x4_t& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(kLeft));
}
template <int kLeft>
__device__ __forceinline__ void lds_wait(u32x2_t& a, u32x2_t& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(kLeft));
}
template <int kLeft>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(kLeft));
}
template <int kLeft>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b, u32x4_t& c, u32x4_t& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(kLeft));
}

// x combined with the value of lane l ^ 32, on the VALU (v_permlane32_swap):
// returns {x[l], x[l ^ 32]} in some order, which is all a symmetric reduction
// needs.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// The same with lane l ^ 16 (v_permlane16_swap: rows 1 and 3 of one copy
// trade places with rows 0 and 2 of the other).
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------- FP8 (E4M3) codes
// Sixteen E4M3 codes -> sixteen bf16 values, element i to element i
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact, every E4M3 value is a
// bf16 value).  lo gets codes 0..7, hi codes 8..15.
template <bool kUpper>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kUpper));
}
__device__ __forceinline__ void fp8x16_to_bf16(u32x4_t x, u32x4_t& lo, u32x4_t& hi) {
  lo = u32x4_t{fp8x2_to_bf16x2<false>(x[0]), fp8x2_to_bf16x2<true>(x[0]),
               fp8x2_to_bf16x2<false>(x[1]), fp8x2_to_bf16x2<true>(x[1])};
  hi = u32x4_t{fp8x2_to_bf16x2<false>(x[2]), fp8x2_to_bf16x2<true>(x[2]),
               fp8x2_to_bf16x2<false>(x[3]), fp8x2_to_bf16x2<true>(x[3])};
}
// Four fp32 values -> four E4M3 codes (byte i = value i): magnitudes above
// 448, the largest finite E4M3 value, are clamped first (the conversion
// itself would give NaN there), then v_cvt_pk_fp8_f32 rounds to nearest
// even.  NaN stays NaN.
__device__ __forceinline__ float fp8_clamp(float x) {
  return fabsf(x) > 448.0f ? copysignf(448.0f, x) : x;
}
__device__ __forceinline__ uint32_t f32x4_to_fp8(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(c), fp8_clamp(d), lo, true);
}

// Calls f(std::integral_constant<int, I>) for I = 0..N-1, so that the index
// can be a template argument (an immediate offset) in the body.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------ 16-B access
__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

}  // namespace pa
