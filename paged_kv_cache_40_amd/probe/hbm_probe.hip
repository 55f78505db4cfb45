// Measurement aid, not part of the attention library: a streaming-read kernel
// that gives the HBM read bandwidth this device actually reaches, reported by
// bench.py beside the specification peak.  Each thread reads 16-byte chunks
// grid-strided over the buffer (non-temporal hint, the same access the decode
// kernel uses for K/V rows) and xors them into one word it stores, so no load
// can be dropped.  Built into libpa_probe.so.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                               int64_t n16, uint32_t* out) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[tid] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device pointer `src`; `out` must hold
// blocks*256 uint32 values.  Returns 0, or -1 if the arguments or the launch fail.
extern "C" int pa_probe_stream_read(const void* src, int64_t bytes, void* out, int32_t blocks,
                                    void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                     static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
