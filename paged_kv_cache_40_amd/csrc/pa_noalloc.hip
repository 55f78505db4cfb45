// pa_decode_noalloc: pa_decode_ext for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).  The decode workspace -
// the per-partition partial results the merge pass combines - lives in a file-scope device
// array of fixed size instead of a caller buffer.  The runtime gives every device that loads
// this library its own copy of the array when it loads the library's code; this file looks up
// each device's address once, with that device current, and passes that address to the same
// kernels pa_decode_ext launches.  Nothing here allocates.
//
// Calls on one device share its array: calls that overlap in time on one device (two streams,
// two threads) race on it.  No kernel needs the array cleared: every partial the merge passes
// read is written by the same call first.

#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.hpp"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_WORKSPACE_BYTES;
static_assert(kScratchBytes % 256 == 0, "the array keeps the workspace's 256-byte alignment");

// In host code this name stands for the device array; only the address looked up below may be
// passed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device the call's work runs on: the stream's, or the current one for the null stream.
int call_device(hipStream_t stream, int* dev) {
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, dev) == hipSuccess) return PA_OK;
    (void)hipGetLastError();
    return PA_ERR_LAUNCH;
  }
  if (hipGetDevice(dev) == hipSuccess) return PA_OK;
  (void)hipGetLastError();
  return PA_ERR_LAUNCH;
}

// Address of device `dev`'s copy of `scratch`, looked up on the first call for that device
// with the device current (the caller's current device is restored afterwards).
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return PA_ERR_LAUNCH;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return PA_ERR_LAUNCH;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_LAUNCH;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* q, const void* k_pool,
                                 const void* v_pool, int64_t num_blocks,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, const int32_t* q_start_loc,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_context_len,
                                 int32_t max_query_len, int32_t num_heads, int32_t head_dim,
                                 int32_t block_size, int32_t dtype, int32_t sliding_window,
                                 const float* alibi_slopes, uint32_t flags, void* stream) {
  pa::DecodeCall c{out, q, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
                   context_lens, q_start_loc, num_seqs, num_tokens, max_context_len,
                   max_query_len, num_heads, head_dim, block_size, dtype, sliding_window,
                   alibi_slopes, flags};
  if (int st = pa::check_decode(c)) return st;
  const size_t need = pa::decode_workspace_bytes(num_tokens, num_heads, head_dim, max_context_len);
  if (need > kScratchBytes) return PA_ERR_WORKSPACE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    if (int e = call_device(st, &dev)) return e;
    if (int e = scratch_on(dev, &ws)) return e;
  }
  return pa::run_decode(c, ws, st);
}
