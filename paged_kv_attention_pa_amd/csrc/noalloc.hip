// pa_decode_noalloc: pa_decode with its workspace taken from a device array
// the library owns, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The kernels are pa_decode's; only where the split partials
// (or the token-balanced segments) live changes.
//
// The array is a file-scope __device__ object: every device the library runs
// on holds its own copy from the first launch on that device until the
// process ends.  In host code its name is a host-side stand-in, so its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and only that address is passed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "pa.h"

namespace {

constexpr size_t kScratchBytes = size_t(PA_NOALLOC_SCRATCH_BYTES);

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first
// call on each device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

pa_status_t pa_decode_noalloc(pa_dtype_t dtype, const void* q, const void* k, const void* v,
                              void* kv_cache, int64_t num_blocks, int block_size,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int64_t* slot_mapping, const int32_t* seq_lens,
                              int num_seqs, int max_seq_len, int num_q_heads, int num_kv_heads,
                              int head_dim, float scale, int num_splits, void* out, float* lse,
                              hipStream_t stream) {
  if (out == nullptr)
    return pa_status_t(pa::set_error(PA_ERR_INVALID,
                                     "pa_decode_noalloc needs out: the partial-only form would "
                                     "leave its partials in the library's own array"));
  size_t need = 0;
  pa_status_t st = pa_decode_workspace_size(dtype, num_seqs, max_seq_len, block_size,
                                            num_q_heads, num_kv_heads, head_dim, num_splits, 0,
                                            &need);
  if (st != PA_OK) return st;
  if (need > kScratchBytes)
    return pa_status_t(pa::set_error(PA_ERR_WORKSPACE,
                                     "pa_decode_noalloc: this batch needs %zu bytes of workspace, "
                                     "the library's array holds %zu (PA_NOALLOC_SCRATCH_BYTES); "
                                     "use pa_decode with a workspace",
                                     need, kScratchBytes));
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess)
      return pa_status_t(pa::set_error(PA_ERR_HIP, "pa_decode_noalloc: scratch array address: %s",
                                       hipGetErrorString(e)));
  }
  return pa_decode(dtype, q, k, v, kv_cache, num_blocks, block_size, block_table,
                   max_blocks_per_seq, slot_mapping, seq_lens, num_seqs, max_seq_len,
                   num_q_heads, num_kv_heads, head_dim, scale, num_splits, ws,
                   need > 0 ? kScratchBytes : 0, out, lse, stream);
}

}  // extern "C"
