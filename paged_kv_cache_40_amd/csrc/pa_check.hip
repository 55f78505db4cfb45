// Device-side precondition checks: the contents of block tables, context lengths, start
// locations and block pairs, which the compute kernels take on trust.
//
// Sources: P1 = "Efficient Memory Management for Large Language Model Serving
// with PagedAttention" (urban-dandelion.tistory.com/4); P2 = "SOSP 2023論文解説:
// vLLM — PagedAttentionによるKVキャッシュメモリ管理の革新".
//
// What is checked [P1 sec. 4, the addressing sentence, and sec. 5, Fig. 7: token j of a
// sequence lives in block_tables[s][j / B], slot j % B; P2 pseudocode: append writes the next
// slot, copy_on_write gives a writer its own copy of a shared block]:
//   attention: start locations 0-based and non-decreasing; 1 <= n_s <= max_query_len;
//     n_s <= L_s <= min(max_blocks * B, max_context_len); the table entries of every block
//     holding a key some query of s attends to lie in [0, num_blocks).
//   write: start locations as above (n_s = 0 allowed); n_s <= L_s <= max_blocks * B; the
//     entries of the written blocks in range; no two written tokens in one slot.
//   pairs: ids inside their pools; destinations distinct; for a copy inside one pool no
//     destination is also a source.
// A violation is reported as (kind << 32) | index into one 64-bit word by atomic minimum, so
// the word holds the smallest kind found and its smallest sequence or pair index, whatever
// the order the threads run in.  Collisions use two bits per slot (or block): the first
// pass sets "seen" and, for a second visitor, "shared"; the second pass reports every
// visitor of a shared slot, the lowest of which the minimum keeps.
// Every load is bounds-checked before use, so malformed inputs cannot fault these kernels.

#include "../../include/pa.h"
#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void report(unsigned long long* err, int kind, int64_t index) {
  atomicMin(err, (static_cast<unsigned long long>(kind) << 32) |
                     static_cast<unsigned long long>(static_cast<uint32_t>(index)));
}

__global__ __launch_bounds__(kThreads) void check_init_kernel(unsigned long long* err,
                                                              uint32_t* marks, int64_t words) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < words;
       i += stride)
    marks[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) *err = ~0ull;
}

// Start locations of sequence s (NULL: one token each).  Returns n_s; flags a broken prefix.
// 64-bit arithmetic throughout: arbitrary device values never overflow.
__device__ __forceinline__ int64_t count_of(const int32_t* loc, int s, int num_seqs,
                                            int num_tokens, unsigned long long* err) {
  if (loc == nullptr) return 1;
  const int64_t a = loc[s], b = loc[s + 1];
  if ((s == 0 && a != 0) || b < a || (s == num_seqs - 1 && b > num_tokens))
    report(err, PA_CHECK_START_LOC, s);
  return b - a;
}

struct AttnCheck {
  unsigned long long* err;
  int64_t num_blocks;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* q_start_loc;
  int32_t max_blocks, num_seqs, num_tokens, max_context_len, max_query_len, block_size, window;
};

// One thread per sequence.
__global__ __launch_bounds__(kThreads) void check_attention_kernel(AttnCheck a) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= a.num_seqs) return;
  const int64_t n = count_of(a.q_start_loc, s, a.num_seqs, a.num_tokens, a.err);
  if (n < 1 || n > a.max_query_len) report(a.err, PA_CHECK_QUERY_COUNT, s);
  const int64_t L = a.context_lens[s];
  const int64_t cap = static_cast<int64_t>(a.max_blocks) * a.block_size;
  if (L < n || L > cap || L > a.max_context_len) report(a.err, PA_CHECK_CONTEXT_LEN, s);
  if (L < 1 || n < 1 || L < n) return;
  // keys any query of s attends to: from the first query's window start to the context end
  const int64_t last = (L > cap ? cap : L) - 1;
  int64_t first = 0;
  if (a.window > 0) {
    const int64_t p0 = L - n;  // the first query's position
    first = p0 - a.window + 1 > 0 ? p0 - a.window + 1 : 0;
  }
  if (first > last) return;
  const int32_t* row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  for (int64_t j = first / a.block_size; j <= last / a.block_size; ++j) {
    const int b = row[j];
    if (b < 0 || b >= a.num_blocks) {
      report(a.err, PA_CHECK_BLOCK_ID, s);
      break;
    }
  }
}

struct WriteCheck {
  unsigned long long* err;
  uint32_t* seen;    // one bit per slot
  uint32_t* shared;  // one bit per slot
  int64_t num_blocks;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* write_start_loc;
  int32_t max_blocks, num_seqs, num_tokens, block_size;
};

// One thread per sequence: start locations and lengths.
__global__ __launch_bounds__(kThreads) void check_write_seq_kernel(WriteCheck a) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= a.num_seqs) return;
  const int64_t n = count_of(a.write_start_loc, s, a.num_seqs, a.num_tokens, a.err);
  const int64_t L = a.context_lens[s];
  if (L < n || L > static_cast<int64_t>(a.max_blocks) * a.block_size)
    report(a.err, PA_CHECK_CONTEXT_LEN, s);
}

// Slot of token row t, or -1 when the row is not written or its position or block is out of
// range (those are reported by kind here or by the per-sequence pass).
__device__ __forceinline__ int64_t slot_of(const WriteCheck& a, int t, int* seq) {
  int s = t;
  int64_t first = t, n = 1;
  if (a.write_start_loc != nullptr) {
    int lo = 0, hi = a.num_seqs - 1;  // largest s with loc[s] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.write_start_loc[mid] <= t) lo = mid; else hi = mid - 1;
    }
    s = lo;
    first = a.write_start_loc[s];
    n = a.write_start_loc[s + 1] - first;
    if (t < first || t - first >= n) return -1;
  }
  *seq = s;
  const int64_t p = a.context_lens[s] - n + (t - first);
  if (p < 0 || p >= static_cast<int64_t>(a.max_blocks) * a.block_size) return -1;
  const int b = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + p / a.block_size];
  if (b < 0 || b >= a.num_blocks) {
    report(a.err, PA_CHECK_BLOCK_ID, s);
    return -1;
  }
  return static_cast<int64_t>(b) * a.block_size + p % a.block_size;
}

// One thread per token row: mark its slot.
__global__ __launch_bounds__(kThreads) void check_write_mark_kernel(WriteCheck a) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= a.num_tokens) return;
  int s = 0;
  const int64_t slot = slot_of(a, t, &s);
  if (slot < 0) return;
  const uint32_t bit = 1u << (slot & 31);
  if (atomicOr(&a.seen[slot >> 5], bit) & bit) atomicOr(&a.shared[slot >> 5], bit);
}

// One thread per token row: every writer of a shared slot reports its sequence.
__global__ __launch_bounds__(kThreads) void check_write_collide_kernel(WriteCheck a) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= a.num_tokens) return;
  int s = 0;
  const int64_t slot = slot_of(a, t, &s);
  if (slot < 0) return;
  if (a.shared[slot >> 5] & (1u << (slot & 31))) report(a.err, PA_CHECK_SLOT_REUSED, s);
}

struct PairCheck {
  unsigned long long* err;
  uint32_t* seen;    // one bit per destination block
  uint32_t* shared;  // one bit per destination block
  int64_t num_src, num_dst;
  const int32_t* pairs;
  int32_t num_pairs, same_pool;
};

// One thread per pair: ids in range, then mark the destination.
__global__ __launch_bounds__(kThreads) void check_pairs_mark_kernel(PairCheck a) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.num_pairs) return;
  const int src = a.pairs[2 * i], dst = a.pairs[2 * i + 1];
  if (src < 0 || src >= a.num_src || dst < 0 || dst >= a.num_dst) {
    report(a.err, PA_CHECK_PAIR_ID, i);
    if (dst < 0 || dst >= a.num_dst) return;
  }
  const uint32_t bit = 1u << (dst & 31);
  if (atomicOr(&a.seen[dst >> 5], bit) & bit) atomicOr(&a.shared[dst >> 5], bit);
}

// One thread per pair: shared destinations; inside one pool, sources that are destinations.
__global__ __launch_bounds__(kThreads) void check_pairs_collide_kernel(PairCheck a) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.num_pairs) return;
  const int src = a.pairs[2 * i], dst = a.pairs[2 * i + 1];
  if (dst >= 0 && dst < a.num_dst && (a.shared[dst >> 5] & (1u << (dst & 31))))
    report(a.err, PA_CHECK_DEST_REUSED, i);
  if (a.same_pool && src >= 0 && src < a.num_dst && (a.seen[src >> 5] & (1u << (src & 31))))
    report(a.err, PA_CHECK_DEST_IS_SOURCE, i);
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + kThreads - 1) / kThreads;
  return static_cast<unsigned>(g < 1 ? 1 : g);
}

hipError_t init(unsigned long long* err, uint32_t* marks, int64_t words, hipStream_t st) {
  int64_t g = (words + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > 1024 ? 1024 : g);
  hipLaunchKernelGGL(check_init_kernel, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, st,
                     err, marks, words);
  return hipGetLastError();
}

}  // namespace

int64_t check_mark_words(int64_t marks) { return (marks + 31) / 32; }

hipError_t launch_check_attention(uint64_t* err, int64_t num_blocks, const int32_t* block_tables,
                                  int32_t max_blocks, const int32_t* context_lens,
                                  const int32_t* q_start_loc, int32_t num_seqs,
                                  int32_t num_tokens, int32_t max_context_len,
                                  int32_t max_query_len, int32_t block_size, int32_t window,
                                  hipStream_t st) {
  auto* e = reinterpret_cast<unsigned long long*>(err);
  hipError_t r = init(e, nullptr, 0, st);
  if (r != hipSuccess) return r;
  AttnCheck a{e, num_blocks, block_tables, context_lens, q_start_loc, max_blocks, num_seqs,
              num_tokens, max_context_len, max_query_len, block_size, window};
  hipLaunchKernelGGL(check_attention_kernel, dim3(grid_for(num_seqs)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_check_write(uint64_t* err, void* workspace, int64_t num_blocks,
                              const int32_t* block_tables, int32_t max_blocks,
                              const int32_t* context_lens, const int32_t* write_start_loc,
                              int32_t num_seqs, int32_t num_tokens, int32_t block_size,
                              hipStream_t st) {
  auto* e = reinterpret_cast<unsigned long long*>(err);
  const int64_t words = check_mark_words(num_blocks * block_size);
  auto* seen = static_cast<uint32_t*>(workspace);
  hipError_t r = init(e, seen, 2 * words, st);
  if (r != hipSuccess) return r;
  WriteCheck a{e, seen, seen + words, num_blocks, block_tables, context_lens, write_start_loc,
               max_blocks, num_seqs, num_tokens, block_size};
  hipLaunchKernelGGL(check_write_seq_kernel, dim3(grid_for(num_seqs)), dim3(kThreads), 0, st, a);
  if (num_tokens > 0) {
    hipLaunchKernelGGL(check_write_mark_kernel, dim3(grid_for(num_tokens)), dim3(kThreads), 0,
                       st, a);
    hipLaunchKernelGGL(check_write_collide_kernel, dim3(grid_for(num_tokens)), dim3(kThreads), 0,
                       st, a);
  }
  return hipGetLastError();
}

hipError_t launch_check_pairs(uint64_t* err, void* workspace, int64_t num_src, int64_t num_dst,
                              const int32_t* pairs, int32_t num_pairs, int32_t same_pool,
                              hipStream_t st) {
  auto* e = reinterpret_cast<unsigned long long*>(err);
  const int64_t words = check_mark_words(num_dst);
  auto* seen = static_cast<uint32_t*>(workspace);
  hipError_t r = init(e, seen, 2 * words, st);
  if (r != hipSuccess || num_pairs == 0) return r;
  PairCheck a{e, seen, seen + words, num_src, num_dst, pairs, num_pairs, same_pool};
  hipLaunchKernelGGL(check_pairs_mark_kernel, dim3(grid_for(num_pairs)), dim3(kThreads), 0, st,
                     a);
  hipLaunchKernelGGL(check_pairs_collide_kernel, dim3(grid_for(num_pairs)), dim3(kThreads), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace pa
