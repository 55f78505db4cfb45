// Host-side launchers behind the C ABI (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// DecodeArgs::flags: neighbouring sequences share blocks (cached loads, XCD-grouped launch)
constexpr uint32_t kDecodeSharedBlocks = 1u;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  const int32_t* q_start_loc;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_heads;
  int32_t block_size;
  int32_t max_context_len; // host bound; device context lengths are clamped to it
  float scale_log2;        // log2(e) / sqrt(head_dim)
  int32_t window;          // sliding window in tokens (0 = none)
  const float* alibi;      // per-head ALiBi slopes [num_heads] or nullptr
  uint32_t flags;          // kDecode* bits
  int32_t group;           // > 1: consecutive runs of this many sequences may share blocks
  void* workspace;         // caller's scratch (see decode_workspace_bytes)
  // set by the launcher:
  const int32_t* order;    // nullptr, or the sequence each grid row of pass 1 takes
                           // (longest context first), in the workspace
  int32_t heads_per_wg;    // waves (one head each) per workgroup
  int32_t num_parts_max;   // partition slots per (query row, head) in the workspace
  int32_t part_size;       // tokens per context partition
  float* ws_acc;           // [num_tokens][num_heads][num_parts_max][head_dim]
  float* ws_ml;            // [num_tokens][num_heads][num_parts_max][2] = (max, sum), log2 domain
};

struct TileArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  const int32_t* q_start_loc;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_heads;
  float scale_log2;
  int32_t window;          // sliding window in tokens (0 = none)
  const float* alibi;      // per-head ALiBi slopes [num_heads] or nullptr
  int32_t block_size;
  // Key splits: a tile whose key steps exceed split_steps is spread over up to splits_max
  // workgroups (the last takes the rest), each writing fp32 partials to the workspace, merged
  // by a second pass.  split_steps = 0: one workgroup per tile.
  int32_t split_steps;
  int32_t splits_max;
  int32_t num_parts_max;   // partition slots per (query row, head) in the workspace
  float* ws_acc;           // [num_tokens][num_heads][num_parts_max][head_dim]
  float* ws_ml;            // [num_tokens][num_heads][num_parts_max][2] = (max, sum), log2 domain
};

// The arguments of one attention call (pa_decode_ext without its workspace), as the C ABI
// received them.
struct DecodeCall {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  const int32_t* q_start_loc;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_context_len;
  int32_t max_query_len;
  int32_t num_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t dtype;
  int32_t sliding_window;
  const float* alibi_slopes;
  uint32_t flags;
};

// Host-side argument checks of an attention call (everything but the workspace): PA_OK or the
// pa_status of the first failure.  No HIP call.
int check_decode(const DecodeCall& c);
// Launch the checked call with a workspace of at least decode_workspace_bytes(...) bytes.
int run_decode(const DecodeCall& c, void* workspace, hipStream_t stream);

// Largest sequence group of the grouped decode (fp16, no window, one query per
// sequence).
constexpr int kMaxDecodeGroup = 6;

// Smallest context partition any decode launch uses; sizes the workspace.
constexpr int kMinPartition = 256;

// Partition slots per (query row, head) in the workspace: one per kMinPartition tokens of the
// longest context.  Decode partitions and tile key splits both index slots with this stride,
// so the slots of different query rows never overlap.
inline int workspace_parts(int max_context_len) {
  return (max_context_len + kMinPartition - 1) / kMinPartition;
}

// Workspace bytes for the partial results of a decode launch (0 when no
// sequence spans more than one partition).
size_t decode_workspace_bytes(int64_t num_tokens, int64_t num_heads, int64_t head_dim,
                              int64_t max_context_len);

// dtype: 0 = fp32, 1 = fp16.  Return hipSuccess or the launch error.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                         int max_context_len, hipStream_t stream);
// a.workspace-derived fields (split_steps .. ws_ml) are set by the launcher.
hipError_t launch_tile(const TileArgs& a, void* workspace, int head_dim, int block_size,
                       int max_query_len, int max_context_len, hipStream_t stream);
hipError_t launch_write_kv(void* k_pool, void* v_pool, int64_t num_blocks, const void* k_new,
                           const void* v_new, const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, const int32_t* write_start_loc,
                           int32_t num_seqs, int32_t num_tokens, int64_t row_bytes,
                           int32_t block_size, hipStream_t stream);
hipError_t launch_swap_blocks(void* dst_k, void* dst_v, int64_t dst_blocks, const void* src_k,
                              const void* src_v, int64_t src_blocks, const int32_t* block_pairs,
                              int32_t num_pairs, int64_t block_bytes, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks,
                              const int32_t* block_pairs, int32_t num_pairs, int64_t block_bytes,
                              hipStream_t stream);

// Device-side precondition checks (pa_check.hip).  err: one 64-bit word; workspace: two
// bitmaps of check_mark_words(n) words each (n = slots for a write, destination blocks for
// pairs).
int64_t check_mark_words(int64_t marks);
hipError_t launch_check_attention(uint64_t* err, int64_t num_blocks, const int32_t* block_tables,
                                  int32_t max_blocks, const int32_t* context_lens,
                                  const int32_t* q_start_loc, int32_t num_seqs,
                                  int32_t num_tokens, int32_t max_context_len,
                                  int32_t max_query_len, int32_t block_size, int32_t window,
                                  hipStream_t stream);
hipError_t launch_check_write(uint64_t* err, void* workspace, int64_t num_blocks,
                              const int32_t* block_tables, int32_t max_blocks,
                              const int32_t* context_lens, const int32_t* write_start_loc,
                              int32_t num_seqs, int32_t num_tokens, int32_t block_size,
                              hipStream_t stream);
hipError_t launch_check_pairs(uint64_t* err, void* workspace, int64_t num_src, int64_t num_dst,
                              const int32_t* pairs, int32_t num_pairs, int32_t same_pool,
                              hipStream_t stream);

}  // namespace pa
