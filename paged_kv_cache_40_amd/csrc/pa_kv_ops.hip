// Slot write and copy-on-write block copy for gfx950.
//
// Sources: P1 = "Efficient Memory Management for Large Language Model Serving
// with PagedAttention" (urban-dandelion.tistory.com/4); P2 = "SOSP 2023論文解説:
// vLLM — PagedAttentionによるKVキャッシュメモリ管理の革新".
//
// write_kv [P2 "アルゴリズムの擬似コード", append_token; P1 sec. 5, Fig. 7]:
//   the i-th of sequence s's n new tokens is at position p = ctx[s] - n + i and
//   its whole token row (all heads) goes to block_tables[s][p / B], slot p % B.
//   A token row is contiguous in both the source [T][H][d] and the pool
//   [NB][B][H][d], so one workgroup streams it with 16-byte loads and stores.
//   blockIdx.y selects K (0) or V (1).
// copy_blocks [P2 pseudocode, copy_on_write; P1 sec. 6, Fig. 9]: a physical
//   block is one contiguous B*H*d run of the pool; each workgroup copies a
//   16 KB slice of one (pair, K-or-V) block with 16-byte accesses.
// swap_blocks [P1 sec. 5, preemption by swapping; P3 "오프로딩"]: whole
//   blocks between the device pool and a host swap pool in pinned memory that
//   the device addresses directly, all pairs in one launch: the host link is
//   driven by the loads and stores of many workgroups at once, each thread
//   keeping four 16-byte transfers in flight.
// All copies are bit-exact: bytes are moved, never converted.  Slots or
// blocks that fall outside the pool (malformed device data) are skipped.

#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

constexpr int kCopyThreads = 256;
constexpr int64_t kCopySlice = 16384;

__device__ __forceinline__ void copy_row(char* dst, const char* src, int64_t bytes) {
  for (int64_t off = static_cast<int64_t>(threadIdx.x) * 16; off < bytes;
       off += static_cast<int64_t>(blockDim.x) * 16)
    st16(dst + off, ld16(src + off));
}

__global__ __launch_bounds__(kCopyThreads) void write_kv_kernel(
    char* k_pool, char* v_pool, int64_t num_blocks, const char* k_new, const char* v_new,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
    const int32_t* write_start_loc, int32_t num_seqs, int32_t num_tokens, int64_t row_bytes,
    int32_t block_size) {
  const int t = blockIdx.x;
  int s = t;
  int64_t first = t, n = 1;  // 64-bit: malformed device values cannot overflow
  if (write_start_loc != nullptr) {
    // largest s with write_start_loc[s] <= t (sequences with no new token are skipped)
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (write_start_loc[mid] <= t) lo = mid; else hi = mid - 1;
    }
    s = lo;
    first = write_start_loc[s];
    n = write_start_loc[s + 1] - first;
    if (t < first || t - first >= n) return;
  }
  const int64_t p = context_lens[s] - n + (t - first);
  if (p < 0 || p >= static_cast<int64_t>(max_blocks) * block_size) return;
  const int blk = block_tables[static_cast<int64_t>(s) * max_blocks + p / block_size];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t dst = (static_cast<int64_t>(blk) * block_size + p % block_size) * row_bytes;
  const int64_t src = static_cast<int64_t>(t) * row_bytes;
  if (blockIdx.y == 0) copy_row(k_pool + dst, k_new + src, row_bytes);
  else copy_row(v_pool + dst, v_new + src, row_bytes);
}

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char* k_pool, char* v_pool, int64_t num_blocks, const int32_t* block_pairs,
    int64_t block_bytes) {
  const int pr = blockIdx.x;
  const int src = block_pairs[2 * pr];
  const int dst = block_pairs[2 * pr + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* pool = blockIdx.z == 0 ? k_pool : v_pool;
  const int64_t lo = static_cast<int64_t>(blockIdx.y) * kCopySlice;
  const int64_t n = min(kCopySlice, block_bytes - lo);
  if (n <= 0) return;
  copy_row(pool + static_cast<int64_t>(dst) * block_bytes + lo,
           pool + static_cast<int64_t>(src) * block_bytes + lo, n);
}

// 16 KB slice per workgroup of 256 threads: four 16-byte loads in flight per thread
// before the stores (a host-link access takes microseconds).
__device__ __forceinline__ void copy_slice_4(char* dst, const char* src, int64_t bytes) {
  constexpr int64_t kStep = kCopyThreads * 16;
  int64_t off = static_cast<int64_t>(threadIdx.x) * 16;
  for (; off + 3 * kStep < bytes; off += 4 * kStep) {
    u32x4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = ld16(src + off + u * kStep);
#pragma unroll
    for (int u = 0; u < 4; ++u) st16(dst + off + u * kStep, r[u]);
  }
  for (; off < bytes; off += kStep) st16(dst + off, ld16(src + off));
}

__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    char* dst_k, char* dst_v, int64_t dst_blocks, const char* src_k, const char* src_v,
    int64_t src_blocks, const int32_t* block_pairs, int64_t block_bytes) {
  const int pr = blockIdx.x;
  const int src = block_pairs[2 * pr];
  const int dst = block_pairs[2 * pr + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const int64_t lo = static_cast<int64_t>(blockIdx.y) * kCopySlice;
  const int64_t n = min(kCopySlice, block_bytes - lo);
  if (n <= 0) return;
  const int64_t so = static_cast<int64_t>(src) * block_bytes + lo;
  const int64_t d_o = static_cast<int64_t>(dst) * block_bytes + lo;
  if (blockIdx.z == 0)
    copy_slice_4(dst_k + d_o, src_k + so, n);
  else
    copy_slice_4(dst_v + d_o, src_v + so, n);
}

hipError_t launch_swap_blocks(void* dst_k, void* dst_v, int64_t dst_blocks, const void* src_k,
                              const void* src_v, int64_t src_blocks, const int32_t* block_pairs,
                              int32_t num_pairs, int64_t block_bytes, hipStream_t stream) {
  dim3 grid(num_pairs, static_cast<unsigned>((block_bytes + kCopySlice - 1) / kCopySlice), 2);
  hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(kCopyThreads), 0, stream,
                     static_cast<char*>(dst_k), static_cast<char*>(dst_v), dst_blocks,
                     static_cast<const char*>(src_k), static_cast<const char*>(src_v), src_blocks,
                     block_pairs, block_bytes);
  return hipGetLastError();
}

hipError_t launch_write_kv(void* k_pool, void* v_pool, int64_t num_blocks, const void* k_new,
                           const void* v_new, const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, const int32_t* write_start_loc,
                           int32_t num_seqs, int32_t num_tokens, int64_t row_bytes,
                           int32_t block_size, hipStream_t stream) {
  dim3 grid(num_tokens, 2);
  hipLaunchKernelGGL(write_kv_kernel, grid, dim3(kCopyThreads), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), num_blocks,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                     block_tables, max_blocks, context_lens, write_start_loc, num_seqs, num_tokens,
                     row_bytes, block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks,
                              const int32_t* block_pairs, int32_t num_pairs, int64_t block_bytes,
                              hipStream_t stream) {
  dim3 grid(num_pairs, static_cast<unsigned>((block_bytes + kCopySlice - 1) / kCopySlice), 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), num_blocks,
                     block_pairs, block_bytes);
  return hipGetLastError();
}

}  // namespace pa
