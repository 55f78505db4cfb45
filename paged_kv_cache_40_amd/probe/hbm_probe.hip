// Measurement aid, not part of the attention library: a streaming-read kernel
// that gives the HBM read bandwidth this device actually reaches, reported by
// bench.py beside the specification peak.  Each workgroup reads whole 256 KB
// chunks of the buffer (chunks dealt to workgroups round-robin), 16 bytes per
// thread per load with the non-temporal hint and eight loads in flight, and
// xors what it reads into one word per thread that it stores, so no load can
// be dropped.  On MI355X this contiguous-chunk pattern reads faster than a
// grid-strided sweep of the whole buffer, so it is the higher (more honest)
// ceiling to compare against.  Built into libpa_probe.so.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int64_t kChunk16 = 16384;  // 16-byte units per chunk (256 KB)
static_assert(kChunk16 % (kThreads * kUnroll) == 0, "chunks hold whole unrolled sweeps");

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                               int64_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const int t = threadIdx.x;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk16; base < n16;
       base += static_cast<int64_t>(gridDim.x) * kChunk16) {
    const int64_t end = base + kChunk16 < n16 ? base + kChunk16 : n16;
    int64_t i = base + t;
    for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += kThreads) {  // ragged end of the last chunk
      const u32x4 v = __builtin_nontemporal_load(p + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  out[static_cast<int64_t>(blockIdx.x) * kThreads + t] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device pointer `src` with `blocks`
// workgroups; `out` must hold blocks*256 uint32 values.  Returns 0, or -1 if the
// arguments or the launch fail.
extern "C" int pa_probe_stream_read(const void* src, int64_t bytes, void* out, int32_t blocks,
                                    void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                     static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
