// C ABI of the paged KV-cache library: host-side argument checks, then the
// launchers.  Every check here runs before any launch, so a rejected call
// touches neither the device nor the stream; only pa_swap_blocks asks the HIP
// runtime (a query, no device work) whether its host pool is mapped memory.

#include <math.h>

#include "../../include/pa.h"
#include "pa_internal.hpp"

namespace {

bool dtype_ok(int32_t dtype) { return dtype == PA_F32 || dtype == PA_F16; }
int elt_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
bool block_size_ok(int32_t b) { return b == 8 || b == 16 || b == 32; }

// Shape checks common to every entry point; returns PA_OK or the first failure.
int check_layout(int64_t num_blocks, int32_t num_heads, int32_t head_dim, int32_t block_size,
                 int32_t dtype) {
  if (num_blocks <= 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0) return PA_ERR_SHAPE;
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || !block_size_ok(block_size))
    return PA_ERR_UNSUPPORTED;
  // a token row (all heads) must be addressable with 32-bit element counts per block
  if (static_cast<int64_t>(num_heads) * head_dim * block_size > (int64_t{1} << 30))
    return PA_ERR_SHAPE;
  return PA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// Device address of a host range [p, p + bytes): both ends must lie in pinned host memory
// mapped for the device, at the same distance apart as on the host; else nullptr.
void* mapped_host_range(void* p, int64_t bytes) {
  void* d0 = nullptr;
  void* d1 = nullptr;
  if (hipHostGetDevicePointer(&d0, p, 0) != hipSuccess || d0 == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  char* last = static_cast<char*>(p) + (bytes - 1);
  if (hipHostGetDevicePointer(&d1, last, 0) != hipSuccess || d1 == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (static_cast<char*>(d1) - static_cast<char*>(d0) != bytes - 1) return nullptr;
  return d0;
}

}  // namespace

namespace pa {

int check_decode(const DecodeCall& c) {
  if (int st = check_layout(c.num_blocks, c.num_heads, c.head_dim, c.block_size, c.dtype))
    return st;
  if (c.sliding_window < 0) return PA_ERR_SHAPE;
  const uint32_t group_bits = 0xFu << PA_DECODE_GROUP_SHIFT;
  if (c.flags & ~(static_cast<uint32_t>(PA_DECODE_SHARED_BLOCKS) | group_bits))
    return PA_ERR_UNSUPPORTED;
  const int group = static_cast<int>((c.flags & group_bits) >> PA_DECODE_GROUP_SHIFT);
  if (group > 1 && (group > kMaxDecodeGroup || (c.flags & PA_DECODE_SHARED_BLOCKS) ||
                    c.dtype != PA_F16 || c.q_start_loc != nullptr || c.sliding_window != 0))
    return PA_ERR_UNSUPPORTED;
  if (c.num_seqs <= 0 || c.num_tokens <= 0 || c.max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (c.max_context_len <= 0 || c.max_query_len <= 0 || c.max_query_len > c.max_context_len)
    return PA_ERR_SHAPE;
  if (static_cast<int64_t>(c.max_context_len) >
      static_cast<int64_t>(c.max_blocks_per_seq) * c.block_size)
    return PA_ERR_SHAPE;
  if (c.q_start_loc == nullptr && (c.num_tokens != c.num_seqs || c.max_query_len != 1))
    return PA_ERR_SHAPE;
  // grid limits of the decode launch: z = sequences, y = context partitions
  if (c.num_seqs > 65535 || c.max_context_len / kMinPartition >= 65535) return PA_ERR_SHAPE;
  // shared-block mode launches one-dimensionally: (head groups x sequences x partitions)
  // workgroups of 256 work-items must stay below 2^32 work-items
  if ((c.flags & PA_DECODE_SHARED_BLOCKS) &&
      static_cast<int64_t>(c.num_heads) * c.num_seqs *
              ((c.max_context_len + kMinPartition - 1) / kMinPartition) >= (int64_t{1} << 24))
    return PA_ERR_SHAPE;
  if (!c.out || !c.q || !c.k_pool || !c.v_pool || !c.block_tables || !c.context_lens)
    return PA_ERR_NULL;
  // the multi-query tile path is built for fp16 (head_dim 64 or 128, as everywhere)
  if (c.max_query_len > 1 && c.dtype != PA_F16) return PA_ERR_UNSUPPORTED;
  if (c.max_query_len > 1 && (c.max_query_len + 63) / 64 > 65535) return PA_ERR_SHAPE;
  return PA_OK;
}

int run_decode(const DecodeCall& c, void* workspace, hipStream_t st) {
  const uint32_t group_bits = 0xFu << PA_DECODE_GROUP_SHIFT;
  const int group = static_cast<int>((c.flags & group_bits) >> PA_DECODE_GROUP_SHIFT);
  DecodeArgs a{};
  a.out = c.out;
  a.q = c.q;
  a.k_pool = c.k_pool;
  a.v_pool = c.v_pool;
  a.num_blocks = c.num_blocks;
  a.block_tables = c.block_tables;
  a.max_blocks = c.max_blocks_per_seq;
  a.context_lens = c.context_lens;
  a.q_start_loc = c.q_start_loc;
  a.num_seqs = c.num_seqs;
  a.num_tokens = c.num_tokens;
  a.num_heads = c.num_heads;
  a.block_size = c.block_size;
  a.max_context_len = c.max_context_len;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(c.head_dim)));
  a.window = c.sliding_window;
  a.alibi = c.alibi_slopes;
  a.flags = c.flags & PA_DECODE_SHARED_BLOCKS;
  a.group = group > 1 ? group : 0;
  a.workspace = workspace;
  // single-query sequences: context partitions + merge; the kernels skip the others
  int status = launch_status(
      launch_decode(a, c.dtype, c.head_dim, c.block_size, c.max_context_len, st));
  if (status != PA_OK || c.max_query_len <= 1) return status;
  // sequences with several queries: causal MFMA tiles
  TileArgs ta{};
  ta.out = c.out;
  ta.q = c.q;
  ta.k_pool = c.k_pool;
  ta.v_pool = c.v_pool;
  ta.num_blocks = c.num_blocks;
  ta.block_tables = c.block_tables;
  ta.max_blocks = c.max_blocks_per_seq;
  ta.context_lens = c.context_lens;
  ta.q_start_loc = c.q_start_loc;
  ta.num_seqs = c.num_seqs;
  ta.num_tokens = c.num_tokens;
  ta.num_heads = c.num_heads;
  ta.scale_log2 = a.scale_log2;
  ta.window = c.sliding_window;
  ta.alibi = c.alibi_slopes;
  return launch_status(launch_tile(ta, workspace, c.head_dim, c.block_size, c.max_query_len,
                                   c.max_context_len, st));
}

}  // namespace pa

extern "C" {

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_ERR_NULL: return "a required pointer argument is NULL";
    case PA_ERR_SHAPE: return "sizes out of range or inconsistent";
    case PA_ERR_UNSUPPORTED: return "dtype, head_dim, block_size or variant not supported";
    case PA_ERR_WORKSPACE: return "workspace missing or smaller than the entry point requires";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_HOST_MEMORY: return "host pool is not pinned host memory mapped for the device";
    default: return "unknown status";
  }
}

size_t pa_decode_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len) {
  if (num_tokens <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  return pa::decode_workspace_bytes(num_tokens, num_heads, head_dim, max_context_len);
}

int pa_write_kv(void* k_pool, void* v_pool, int64_t num_blocks, const void* k_new,
                const void* v_new, const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, const int32_t* write_start_loc, int32_t num_seqs,
                int32_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t block_size,
                int32_t dtype, void* stream) {
  if (int st = check_layout(num_blocks, num_heads, head_dim, block_size, dtype)) return st;
  if (num_seqs <= 0 || num_tokens < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (write_start_loc == nullptr && num_tokens != num_seqs) return PA_ERR_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !context_lens) return PA_ERR_NULL;
  const int64_t row_bytes = static_cast<int64_t>(num_heads) * head_dim * elt_bytes(dtype);
  return launch_status(pa::launch_write_kv(
      k_pool, v_pool, num_blocks, k_new, v_new, block_tables, max_blocks_per_seq, context_lens,
      write_start_loc, num_seqs, num_tokens, row_bytes, block_size,
      static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks, const int32_t* block_pairs,
                   int32_t num_pairs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, void* stream) {
  if (int st = check_layout(num_blocks, num_heads, head_dim, block_size, dtype)) return st;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_pairs) return PA_ERR_NULL;
  const int64_t block_bytes =
      static_cast<int64_t>(block_size) * num_heads * head_dim * elt_bytes(dtype);
  return launch_status(pa::launch_copy_blocks(k_pool, v_pool, num_blocks, block_pairs, num_pairs,
                                              block_bytes, static_cast<hipStream_t>(stream)));
}

int pa_swap_blocks(void* dev_k, void* dev_v, int64_t num_dev_blocks, void* host_k,
                   void* host_v, int64_t num_host_blocks, const int32_t* block_pairs,
                   int32_t num_pairs, int32_t direction, int32_t num_heads, int32_t head_dim,
                   int32_t block_size, int32_t dtype, void* stream) {
  if (int st = check_layout(num_dev_blocks, num_heads, head_dim, block_size, dtype)) return st;
  if (num_host_blocks <= 0 || num_pairs < 0) return PA_ERR_SHAPE;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dev_k || !dev_v || !host_k || !host_v || !block_pairs) return PA_ERR_NULL;
  const int64_t block_bytes =
      static_cast<int64_t>(block_size) * num_heads * head_dim * elt_bytes(dtype);
  if (num_host_blocks > INT64_MAX / block_bytes) return PA_ERR_SHAPE;
  void* hk = mapped_host_range(host_k, num_host_blocks * block_bytes);
  void* hv = mapped_host_range(host_v, num_host_blocks * block_bytes);
  if (hk == nullptr || hv == nullptr) return PA_ERR_HOST_MEMORY;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (direction == PA_SWAP_OUT)
    return launch_status(pa::launch_swap_blocks(hk, hv, num_host_blocks, dev_k, dev_v,
                                                num_dev_blocks, block_pairs, num_pairs,
                                                block_bytes, s));
  return launch_status(pa::launch_swap_blocks(dev_k, dev_v, num_dev_blocks, hk, hv,
                                              num_host_blocks, block_pairs, num_pairs,
                                              block_bytes, s));
}

int pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
              int64_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, const int32_t* q_start_loc, int32_t num_seqs,
              int32_t num_tokens, int32_t max_context_len, int32_t max_query_len,
              int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
              void* workspace, size_t workspace_bytes, void* stream) {
  return pa_decode_ext(out, q, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
                       context_lens, q_start_loc, num_seqs, num_tokens, max_context_len,
                       max_query_len, num_heads, head_dim, block_size, dtype, workspace,
                       workspace_bytes, 0, nullptr, 0, stream);
}

int pa_decode_ext(void* out, const void* q, const void* k_pool, const void* v_pool,
                  int64_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, const int32_t* q_start_loc, int32_t num_seqs,
                  int32_t num_tokens, int32_t max_context_len, int32_t max_query_len,
                  int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                  void* workspace, size_t workspace_bytes, int32_t sliding_window,
                  const float* alibi_slopes, uint32_t flags, void* stream) {
  pa::DecodeCall c{out, q, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
                   context_lens, q_start_loc, num_seqs, num_tokens, max_context_len,
                   max_query_len, num_heads, head_dim, block_size, dtype, sliding_window,
                   alibi_slopes, flags};
  if (int st = pa::check_decode(c)) return st;
  const size_t need = pa::decode_workspace_bytes(num_tokens, num_heads, head_dim, max_context_len);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  return pa::run_decode(c, workspace, static_cast<hipStream_t>(stream));
}

size_t pa_check_workspace_bytes(int64_t num_marks) {
  if (num_marks <= 0) return 0;
  return static_cast<size_t>(2 * pa::check_mark_words(num_marks) * 4);
}

int pa_check_attention(uint64_t* error_word, int64_t num_blocks, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* q_start_loc, int32_t num_seqs, int32_t num_tokens,
                       int32_t max_context_len, int32_t max_query_len, int32_t block_size,
                       int32_t sliding_window, void* stream) {
  if (num_blocks <= 0 || num_seqs <= 0 || num_tokens <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (max_context_len <= 0 || max_query_len <= 0 || sliding_window < 0) return PA_ERR_SHAPE;
  if (q_start_loc == nullptr && num_tokens != num_seqs) return PA_ERR_SHAPE;
  if (!error_word || !block_tables || !context_lens) return PA_ERR_NULL;
  return launch_status(pa::launch_check_attention(
      error_word, num_blocks, block_tables, max_blocks_per_seq, context_lens, q_start_loc,
      num_seqs, num_tokens, max_context_len, max_query_len, block_size, sliding_window,
      static_cast<hipStream_t>(stream)));
}

int pa_check_write(uint64_t* error_word, void* workspace, size_t workspace_bytes,
                   int64_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, const int32_t* write_start_loc, int32_t num_seqs,
                   int32_t num_tokens, int32_t block_size, void* stream) {
  if (num_blocks <= 0 || num_seqs <= 0 || num_tokens < 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (write_start_loc == nullptr && num_tokens != num_seqs) return PA_ERR_SHAPE;
  if (num_blocks > INT64_MAX / block_size) return PA_ERR_SHAPE;
  if (!error_word || !block_tables || !context_lens) return PA_ERR_NULL;
  if (workspace == nullptr || workspace_bytes < pa_check_workspace_bytes(num_blocks * block_size))
    return PA_ERR_WORKSPACE;
  return launch_status(pa::launch_check_write(error_word, workspace, num_blocks, block_tables,
                                              max_blocks_per_seq, context_lens, write_start_loc,
                                              num_seqs, num_tokens, block_size,
                                              static_cast<hipStream_t>(stream)));
}

int pa_check_pairs(uint64_t* error_word, void* workspace, size_t workspace_bytes,
                   int64_t num_src_blocks, int64_t num_dst_blocks, const int32_t* block_pairs,
                   int32_t num_pairs, int32_t same_pool, void* stream) {
  if (num_src_blocks <= 0 || num_dst_blocks <= 0 || num_pairs < 0) return PA_ERR_SHAPE;
  if (same_pool != 0 && same_pool != 1) return PA_ERR_SHAPE;
  if (same_pool && num_src_blocks != num_dst_blocks) return PA_ERR_SHAPE;
  if (!error_word || (num_pairs > 0 && !block_pairs)) return PA_ERR_NULL;
  if (workspace == nullptr || workspace_bytes < pa_check_workspace_bytes(num_dst_blocks))
    return PA_ERR_WORKSPACE;
  return launch_status(pa::launch_check_pairs(error_word, workspace, num_src_blocks,
                                              num_dst_blocks, block_pairs, num_pairs, same_pool,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
