/*
 * pa.h — C ABI of the paged KV-cache attention library (MI355X / gfx950).
 *
 * Sources cited below:
 *   P1 = "Efficient Memory Management for Large Language Model Serving with
 *         PagedAttention" (paper review, urban-dandelion.tistory.com/4)
 *   P2 = "SOSP 2023論文解説: vLLM — PagedAttentionによるKVキャッシュメモリ管理の革新"
 *         (0h-n0.github.io/posts/conf-vllm-pagedattention)
 *   P3 = "연속 배치 처리 아키텍처" (Transformers docs, continuous batching architecture)
 *
 * Conventions shared by every entry point
 *   - Every pointer except the names given as host values (and pa_swap_blocks'
 *     host pool) is DEVICE memory,
 *     owned by the caller; the library keeps no pointer after returning, keeps
 *     no state between calls and allocates nothing.  Calls are thread-safe.
 *   - Tensors are dense, row-major, contiguous.
 *   - K/V pools: k_pool and v_pool, each [num_blocks][block_size][num_heads][head_dim]
 *     elements of `dtype`: one physical block holds block_size token rows, a
 *     token row holds every head's head_dim vector (the per-block
 *     (block_size, num_heads, head_dim) tensor of P2, pseudocode section).
 *     Byte offsets are computed in 64 bits; pools may exceed 2^31 bytes.
 *   - block_tables: int32 [num_seqs][max_blocks_per_seq]; entry b of row s is
 *     the physical block holding tokens b*block_size .. b*block_size+block_size-1
 *     of sequence s (P1 sec. 4, addressing sentence after the attention
 *     equation; P1 sec. 5, Fig. 7).  Entries past the last used one are never
 *     read (the Python side pads with -1).
 *   - context_lens: int32 [num_seqs]; tokens in each sequence INCLUDING the
 *     tokens of the current step (the attention sums run up to the query's own
 *     position, P1 sec. 4 attention equation).
 *   - Start-location arrays (q_start_loc, write_start_loc): int32 [num_seqs+1],
 *     exclusive prefix sums of per-sequence token counts; row r of a
 *     [num_tokens][...] tensor belongs to sequence s when
 *     loc[s] <= r < loc[s+1].  NULL means one token per sequence
 *     (num_tokens == num_seqs, row s belongs to sequence s).  The n tokens of
 *     sequence s are its last n: token i sits at position context_lens[s]-n+i.
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on it and returns; nothing synchronises.
 *   - Supported shapes: dtype PA_F32 or PA_F16, head_dim 64 or 128,
 *     block_size 8, 16 or 32, num_heads >= 1.
 *   - Errors: problems visible from the host arguments return a negative
 *     pa_status and launch nothing.  A failed launch returns PA_ERR_LAUNCH.
 *     Device-resident contents are preconditions, not checked:
 *     1 <= n_s <= context_lens[s] <= max_blocks_per_seq*block_size, table
 *     entries of used blocks in [0, num_blocks), copy destinations distinct and
 *     never a source.  The kernels clamp or skip anything that would address
 *     memory outside the buffers described here, so a violated precondition
 *     gives unspecified values, never an out-of-bounds access: attention
 *     clamps context lengths to the table width (single-query sequences
 *     also to max_context_len), skips a sequence whose length is below 1
 *     or below its query count and reads block 0 in place of an
 *     out-of-range block id; writes skip slots at negative or out-of-table
 *     positions and in out-of-range blocks; copies skip pairs with an
 *     out-of-range id.  Out-of-range ids and lengths of one sequence
 *     therefore change only that sequence's outputs and its own blocks.
 */
#ifndef PAGED_KV_PA_H
#define PAGED_KV_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  PA_ERR_SHAPE = -2,       /* sizes out of range or inconsistent              */
  PA_ERR_UNSUPPORTED = -3, /* dtype / head_dim / block_size / variant not built */
  PA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required         */
  PA_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch        */
  PA_ERR_HOST_MEMORY = -6  /* host pool not pinned memory mapped for the device */
} pa_status;

typedef enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 } pa_swap_direction;

/* pa_decode_ext flags */
typedef enum { PA_DECODE_SHARED_BLOCKS = 1, PA_DECODE_GROUP_SHIFT = 8 } pa_decode_flags;
/* group size g (2..6) for the grouped decode, in flag bits 8..11 */
#define PA_DECODE_GROUP(g) ((uint32_t)(g) << PA_DECODE_GROUP_SHIFT)

/*
 * pa_write_kv — store this step's new K/V rows into their cache slots.
 * Defined by the append step of the block manager (P2, pseudocode section:
 * the new token's K and V go into the next slot of the last block) with the
 * slot given by the block table (P1 sec. 5, Fig. 7).
 *
 * For every row t of k_new / v_new ([num_tokens][num_heads][head_dim] of
 * dtype), belonging to sequence s as its i-th of n new tokens, position
 * p = context_lens[s] - n + i is written to
 *     k_pool[block_tables[s][p / block_size]][p % block_size][:][:]   (and v_pool)
 * The copy is bit-exact.  Rows of different tokens must map to different
 * slots (they do whenever the tables come from a block manager).
 * num_tokens == 0 is a no-op.
 */
int pa_write_kv(void* k_pool, void* v_pool, int64_t num_blocks,
                const void* k_new, const void* v_new,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, const int32_t* write_start_loc,
                int32_t num_seqs, int32_t num_tokens,
                int32_t num_heads, int32_t head_dim, int32_t block_size,
                int32_t dtype, void* stream);

/*
 * pa_decode_workspace_bytes — bytes of device workspace pa_decode needs for
 * a batch whose longest context is max_context_len (0 when no sequence is
 * split into more than one context partition): the partial results of split
 * contexts, then room for the order in which a large launch dispatches its
 * sequences.  Host-only, never fails.
 */
size_t pa_decode_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len);

/*
 * pa_decode — paged attention: for every query row t (sequence s, position p)
 * and head h,
 *     out[t][h][:] = sum_{j<=p} softmax_j(q[t][h]·K_j[h] / sqrt(head_dim)) V_j[h]
 * where K_j, V_j are token j's rows fetched through the block table
 * (P1 sec. 4, attention equation and addressing; P2 section
 * "PagedAttentionの仕組み", blockwise equation computed with online softmax).
 * The scale is fixed at 1/sqrt(head_dim).
 *
 * q, out: [num_tokens][num_heads][head_dim] of dtype (out written in dtype,
 *   rounded to nearest even from fp32 accumulation).
 * q_start_loc: NULL for pure decode (one query per sequence); otherwise
 *   sequences with n_s > 1 queries run the causal multi-query tile path
 *   (chunked prefill mixed with decodes in one batch, P3 section
 *   "Chunked prefill"), each query attending to positions <= its own.
 * max_context_len, max_query_len: host copies of the maxima over the batch
 *   (grid sizing); max_query_len > 1 requires dtype PA_F16 (head_dim 64 or 128).
 * workspace: device scratch of at least
 *   pa_decode_workspace_bytes(num_tokens, num_heads, head_dim, max_context_len)
 *   bytes (NULL allowed when that is 0); contents on return are unspecified.
 */
int pa_decode(void* out, const void* q,
              const void* k_pool, const void* v_pool, int64_t num_blocks,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, const int32_t* q_start_loc,
              int32_t num_seqs, int32_t num_tokens,
              int32_t max_context_len, int32_t max_query_len,
              int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_ext — pa_decode with the two attention variants the block indexing
 * has to accommodate (P1 sec. 10, limitations: sliding-window attention and
 * ALiBi; P3 "메모리 관리": sliding layers keep a fixed window of the most
 * recent tokens).  The pages give no formulas; the readings implemented:
 *   sliding_window W > 0: the query at position p attends to tokens
 *     p-W+1 .. p only (W = 0: no window).  Older tokens never contribute, and
 *     the table entries of blocks that hold only tokens older than every
 *     query's window may be -1: the single-query path never looks them up;
 *     the multi-query path may look up the entries of the (at most three)
 *     such blocks inside the 32-token step where a chunk's window starts,
 *     fetches the named block (block 0 for an invalid entry) and discards
 *     those rows.
 *   alibi_slopes: device float [num_heads] or NULL; slope_h * (j - p) is added
 *     to the score q.k_j / sqrt(head_dim) of token j (0 for the query itself,
 *     more negative with distance).
 * flags: 0, or PA_DECODE_SHARED_BLOCKS when neighbouring sequences of the
 *   batch share blocks (the samples of one prompt, the beams of one search,
 *   requests with a cached common prefix, placed next to each other): the
 *   single-query kernels then keep K/V rows cached and run neighbouring
 *   sequences on the same die, so shared blocks are fetched from HBM about
 *   once (P1 sec. 6: shared blocks are what parallel sampling, beam search
 *   and shared prefixes save).  Results are bit-identical either way; only
 *   speed differs.  Unknown bits return PA_ERR_UNSUPPORTED; with the flag,
 *   num_heads * num_seqs * ceil(max_context_len / 256) must stay below 2^24
 *   (PA_ERR_SHAPE).
 *   PA_DECODE_GROUP(g), g = 2..6, instead: sequences come in runs of g
 *   (sequences 0..g-1, g..2g-1, ..., the last run possibly shorter) whose
 *   members may share their leading blocks, as the samples of one prompt or
 *   the beams of one search do.  Where every member of a run holds the same
 *   physical blocks at the same positions, those K/V rows are read once for
 *   the whole run (P1 sec. 6).  The result is the same attention whatever the
 *   tables hold (the runs only say where to look for sharing); the context
 *   partitions differ from the plain kernel's, so outputs agree with it within
 *   rounding, not bit for bit.  Built for dtype PA_F16 with q_start_loc NULL
 *   and sliding_window 0 (ALiBi slopes allowed), and not combined with
 *   PA_DECODE_SHARED_BLOCKS: other uses return PA_ERR_UNSUPPORTED.  g = 0 or 1
 *   means no runs.  Choosing between the two: the grouped decode needs enough
 *   runs x heads to fill the GPU; below about 1,536 units of
 *   ceil(num_seqs / g) * num_heads * ceil(max_context_len / 256) the
 *   shared-blocks hint is usually faster.
 * pa_decode(...) is pa_decode_ext(..., 0, NULL, 0, stream).  Both variants
 * apply to every query row, single-query decodes and multi-query chunks alike
 * (a chunk's query at position p sees its own window p-W+1 .. p).
 * sliding_window < 0 returns PA_ERR_SHAPE.  The workspace requirement is
 * unchanged.
 */
int pa_decode_ext(void* out, const void* q,
                  const void* k_pool, const void* v_pool, int64_t num_blocks,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, const int32_t* q_start_loc,
                  int32_t num_seqs, int32_t num_tokens,
                  int32_t max_context_len, int32_t max_query_len,
                  int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                  void* workspace, size_t workspace_bytes,
                  int32_t sliding_window, const float* alibi_slopes, uint32_t flags,
                  void* stream);

/*
 * pa_decode_noalloc — pa_decode_ext for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, checks and results as pa_decode_ext, without
 * the workspace: the partial results live in a device array inside the library
 * (PA_NOALLOC_WORKSPACE_BYTES per device that loads it, held until the process
 * ends).  The call allocates nothing and launches the same kernels.
 *   A batch whose pa_decode_workspace_bytes(...) exceeds
 *   PA_NOALLOC_WORKSPACE_BYTES returns PA_ERR_WORKSPACE and launches nothing
 *   (for example 256 sequences x 40 heads x head_dim 128 fit up to contexts of
 *   about 12,800 tokens; chunk query rows count as rows).
 *   The first call on a device looks up that device's array address (a HIP
 *   runtime query, with the stream's device made current for it and the
 *   caller's current device restored); a failed lookup returns PA_ERR_LAUNCH.
 *   Every call on one device shares its array: calls that may overlap in time
 *   on one device (several streams or threads) race and must be serialised by
 *   the caller.  The array needs no clearing between calls.
 */
#define PA_NOALLOC_WORKSPACE_BYTES ((size_t)256 << 20)

int pa_decode_noalloc(void* out, const void* q,
                      const void* k_pool, const void* v_pool, int64_t num_blocks,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, const int32_t* q_start_loc,
                      int32_t num_seqs, int32_t num_tokens,
                      int32_t max_context_len, int32_t max_query_len,
                      int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                      int32_t sliding_window, const float* alibi_slopes, uint32_t flags,
                      void* stream);

/*
 * pa_copy_blocks — copy-on-write block copies, batched: for every pair
 * (src, dst) of block_pairs (int32 [num_pairs][2], device), the whole block
 * k_pool[dst] = k_pool[src] and v_pool[dst] = v_pool[src], every slot filled
 * or not, bit-exact (P2 pseudocode: copy_on_write copies the block's K and V
 * tensors; P1 sec. 6, Fig. 9).  Destinations must be distinct and no
 * destination may be a source.  num_pairs == 0 is a no-op.
 */
int pa_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks,
                   const int32_t* block_pairs, int32_t num_pairs,
                   int32_t num_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, void* stream);

/*
 * pa_swap_blocks — move whole blocks between the device pools and a host swap
 * pool, all pairs in one launch (P1 sec. 5: under memory pressure a preempted
 * sequence's KV blocks are swapped to CPU memory and restored later; P3
 * "오프로딩": offloaded requests' blocks are copied into a pre-allocated pinned
 * CPU buffer in one batched transfer and copied back on resume, nothing
 * recomputed).
 *   dev_k, dev_v: the device pools, num_dev_blocks blocks each (layout above).
 *   host_k, host_v: HOST pointers to the swap pool, num_host_blocks blocks of
 *     the same layout each, in pinned host memory mapped for the device
 *     (hipHostMalloc, or torch tensors made with pin_memory=True).  Pageable
 *     or registered-elsewhere memory returns PA_ERR_HOST_MEMORY; this is the
 *     one check that queries the HIP runtime (no device work).
 *   block_pairs: int32 [num_pairs][2] (src, dst), DEVICE memory.
 *   direction PA_SWAP_OUT: host[dst] = dev[src] (K and V);
 *             PA_SWAP_IN:  dev[dst] = host[src].
 * Whole blocks are copied bit-exact, every slot filled or not.  Destinations
 * must be distinct.  num_pairs == 0 is a no-op.  The copy is ordered on
 * `stream` like every other call: a swap-out must be enqueued before anything
 * that overwrites its source blocks, and the host may read the swap pool only
 * after the stream has been synchronised.  Pairs outside either pool are
 * skipped by the kernel.
 */
int pa_swap_blocks(void* dev_k, void* dev_v, int64_t num_dev_blocks,
                   void* host_k, void* host_v, int64_t num_host_blocks,
                   const int32_t* block_pairs, int32_t num_pairs, int32_t direction,
                   int32_t num_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, void* stream);

/*
 * Precondition checks — the device-resident contents every call above takes on
 * trust (Errors, under the conventions), checked on the device for the same
 * arguments a call would get.  For debugging and for callers that build tables
 * from untrusted input; a serving loop built on the block manager does not
 * need them.  What is checked follows from the addressing the calls implement
 * (P1 sec. 4, the addressing sentence after the attention equation; P1 sec. 5,
 * Fig. 7: token j of sequence s sits in block block_tables[s][j / block_size],
 * slot j % block_size) and from copy-on-write (P2 pseudocode: copy_on_write
 * gives the writer its own block; P1 sec. 6, Fig. 9).
 *
 * error_word: ONE uint64 in device memory, owned by the caller.  Each check
 *   first sets it to PA_CHECK_OK (all ones), then every violation found lowers
 *   it by atomic minimum to (kind << 32) | index, index being the sequence (or
 *   pair) number.  On completion the word holds the smallest kind found and,
 *   for that kind, the smallest index: the same inputs always give the same
 *   word.  Read it after synchronising the stream.
 * workspace (pa_check_write, pa_check_pairs): device scratch of at least
 *   pa_check_workspace_bytes(n) bytes, n = num_blocks * block_size (write) or
 *   num_dst_blocks (pairs); contents on return unspecified.
 * Host arguments are validated as for the calls themselves (negative status,
 * nothing launched).  The checks read only inside the arrays described, so
 * they are safe on any contents.  They enqueue on `stream` and return.
 */
#define PA_CHECK_OK 0xFFFFFFFFFFFFFFFFull

typedef enum {
  PA_CHECK_START_LOC = 1,       /* start locations not 0-based, decreasing, or last > num_tokens */
  PA_CHECK_QUERY_COUNT = 2,     /* attention: n_s < 1 or n_s > max_query_len                      */
  PA_CHECK_CONTEXT_LEN = 3,     /* context_lens[s] < n_s, > max_blocks_per_seq*block_size, or
                                   (attention) > max_context_len                                  */
  PA_CHECK_BLOCK_ID = 4,        /* a table entry the call uses is outside [0, num_blocks)         */
  PA_CHECK_SLOT_REUSED = 5,     /* write: tokens of this sequence share a slot with another token */
  PA_CHECK_PAIR_ID = 6,         /* pairs: src or dst outside its pool                             */
  PA_CHECK_DEST_REUSED = 7,     /* pairs: this pair's destination is another pair's destination   */
  PA_CHECK_DEST_IS_SOURCE = 8   /* pairs in one pool: this pair's source is some pair's destination */
} pa_check_kind;

/* pa_check_workspace_bytes — scratch for n marks (two bits each); 0 when n <= 0. */
size_t pa_check_workspace_bytes(int64_t num_marks);

/*
 * pa_check_attention — the device preconditions of pa_decode / pa_decode_ext
 * with these arguments: start locations, 1 <= n_s <= max_query_len,
 * n_s <= context_lens[s] <= min(max_blocks_per_seq*block_size, max_context_len),
 * and every table entry whose block holds a key some query of s attends to
 * (with sliding_window W > 0, keys from position context_lens[s]-n_s-W+1 on)
 * in [0, num_blocks).
 */
int pa_check_attention(uint64_t* error_word, int64_t num_blocks,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, const int32_t* q_start_loc,
                       int32_t num_seqs, int32_t num_tokens,
                       int32_t max_context_len, int32_t max_query_len,
                       int32_t block_size, int32_t sliding_window, void* stream);

/*
 * pa_check_write — the device preconditions of pa_write_kv: start locations
 * (n_s = 0 allowed), n_s <= context_lens[s] <= max_blocks_per_seq*block_size,
 * the table entries of the written positions in [0, num_blocks), and no two
 * written tokens in one slot (every writer of a shared slot is reported).
 */
int pa_check_write(uint64_t* error_word, void* workspace, size_t workspace_bytes,
                   int64_t num_blocks, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                   const int32_t* write_start_loc, int32_t num_seqs, int32_t num_tokens,
                   int32_t block_size, void* stream);

/*
 * pa_check_pairs — the device preconditions of pa_copy_blocks (same_pool = 1,
 * num_src_blocks == num_dst_blocks == num_blocks) or pa_swap_blocks
 * (same_pool = 0; source and destination pools sized separately): ids inside
 * their pools, destinations distinct (every pair of a shared destination is
 * reported) and, inside one pool, no source that is also a destination.
 */
int pa_check_pairs(uint64_t* error_word, void* workspace, size_t workspace_bytes,
                   int64_t num_src_blocks, int64_t num_dst_blocks,
                   const int32_t* block_pairs, int32_t num_pairs, int32_t same_pool,
                   void* stream);

/* pa_strerror — static text for a pa_status value (never NULL). */
const char* pa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_H */
