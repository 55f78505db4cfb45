// Multi-query (chunked-prefill) paged attention on gfx950 matrix cores.
//
// Sources: P1 = "Efficient Memory Management for Large Language Model Serving
// with PagedAttention" (urban-dandelion.tistory.com/4); P2 = "SOSP 2023論文解説:
// vLLM — PagedAttentionによるKVキャッシュメモリ管理の革新"; P3 = "연속 배치 처리
// 아키텍처" (Transformers docs).
//
// What is computed: for a sequence whose current step carries n > 1 query
// tokens (a prefill chunk, P3 "Chunked prefill"), query i sits at position
// p = ctx - n + i and attends causally to keys 0..p of the same sequence
// [P1 sec. 4, attention equation: sums up to j = i], with keys and values
// fetched through the block table [P1 sec. 4 addressing; Fig. 7].  Prefill is
// matrix-matrix work [P1 sec. 2], so the scores and the value sum run on MFMA.
//
// One workgroup = 4 waves = 64 consecutive queries of one (sequence, head);
// wave w owns queries q0+16w .. q0+16w+15.  Per 16-key block (one paged block
// when B = 16; B = 8 / 32 blocks are split / paired by key index):
//   * the workgroup stages K (row-major, padded rows) and V (transposed,
//     [dim][key]) into LDS, double-buffered, one barrier per block;
//   * each wave computes S^T = K . Q^T (16 keys x 16 queries) with four
//     v_mfma_f32_16x16x32_f16 over head_dim 128; lane (g, r) = (l/16, l%16)
//     holds S^T[key 4g+i][query r], so every per-query quantity lives in the
//     lanes of one column;
//   * causal / context masking by absolute key position, log2-domain online
//     softmax with a running reference that moves only past a 2^8 margin,
//     P^T rounded to fp16 — already the B operand layout of the next product;
//   * O^T += V^T . P^T with eight v_mfma_f32_16x16x16_f16 (16 dims each), V^T
//     read from LDS.
// The denominator sums the same fp16-rounded P values the matrix product uses.
// Values of keys at or past the context length are zeroed when staged (those
// pool slots may hold anything), keys past a query's position are masked.

#include <math.h>

#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

constexpr int kTileQ = 64;       // queries per workgroup
constexpr int kKeys = 16;        // keys per step
constexpr int kD = 128;          // head dim of the tile path
constexpr int kKRow = kD + 8;    // K row stride in LDS (halves): 272 bytes, spreads banks
constexpr int kVRow = kKeys + 4; // V^T row stride in LDS (halves): 40 bytes
constexpr int kKBuf = kKeys * kKRow;  // halves per K buffer
constexpr int kVBuf = kD * kVRow;     // halves per V^T buffer

typedef float f32x4v __attribute__((ext_vector_type(4)));

}  // namespace

template <int BS>
__global__ __launch_bounds__(256) void tile_attention_kernel(TileArgs a) {
  __shared__ __attribute__((aligned(16))) f16 lds_k[2][kKBuf];
  __shared__ __attribute__((aligned(16))) f16 lds_v[2][kVBuf];

  const int h = blockIdx.x;
  const int tile = blockIdx.y;
  const int s = blockIdx.z;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int l = t & 63;
  const int lg = l >> 4;  // lane group 0..3
  const int lr = l & 15;  // column: query within the wave's 16

  const int q_first = a.q_start_loc[s];
  const int n = a.q_start_loc[s + 1] - q_first;
  if (n <= 1) return;  // single-query sequences run the decode path
  const int q0 = tile * kTileQ;
  if (q0 >= n) return;
  const int ctx = min(a.context_lens[s], a.max_blocks * BS);
  if (n > ctx || q_first < 0 || q_first + n > a.num_tokens) return;

  // this lane's query and its absolute position (-1 = no query: fully masked)
  const int q = q0 + 16 * w + lr;
  const int pos = q < n ? ctx - n + q : -1;
  // last key any query of the workgroup / of this wave needs
  const int wg_last = ctx - n + min(q0 + kTileQ - 1, n - 1);
  const int wave_last = ctx - n + min(q0 + 16 * w + 15, n - 1);
  const int nkb = wg_last / kKeys + 1;

  // Q^T operand: lane (lg, lr) holds dims 8*lg + 32*st .. +7 of its query, st = 0..3
  f16x8 qop[4];
  {
    const f16* qp = static_cast<const f16*>(a.q) +
                    (static_cast<int64_t>(q_first + min(q, n - 1)) * a.num_heads + h) * kD;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4 v = ld16(qp + 8 * lg + 32 * st);
      if (q >= n) v = u32x4{0, 0, 0, 0};
      qop[st] = __builtin_bit_cast(f16x8, v);
    }
  }

  const int64_t row_stride = static_cast<int64_t>(a.num_heads) * kD;
  const f16* kpool = static_cast<const f16*>(a.k_pool) + static_cast<int64_t>(h) * kD;
  const f16* vpool = static_cast<const f16*>(a.v_pool) + static_cast<int64_t>(h) * kD;
  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;

  // staging assignment: K: thread -> (key t/16, 16-byte chunk t%16);
  // V: thread -> (key pair t/32, dims 4*(t%32) .. +3) as two 8-byte loads
  const int k_key = t >> 4, k_chunk = t & 15;
  const int v_pair = t >> 5, v_quad = t & 31;
  auto key_row = [&](int key) -> int64_t {  // pool row offset of absolute key `key`
    int blk = btrow[key / BS];
    blk = (blk >= 0 && blk < a.num_blocks) ? blk : 0;
    return (static_cast<int64_t>(blk) * BS + key % BS) * row_stride;
  };
  u32x4 k_reg;
  uint64_t v_reg0, v_reg1;
  auto fetch = [&](int kb) {
    const int key = kb * kKeys + k_key;
    k_reg = ld16(kpool + key_row(min(key, ctx - 1)) + 8 * k_chunk);
    const int key0 = kb * kKeys + 2 * v_pair;
    const int key1 = key0 + 1;
    v_reg0 = *reinterpret_cast<const uint64_t*>(vpool + key_row(min(key0, ctx - 1)) + 4 * v_quad);
    v_reg1 = *reinterpret_cast<const uint64_t*>(vpool + key_row(min(key1, ctx - 1)) + 4 * v_quad);
    if (key0 >= ctx) v_reg0 = 0;  // keys past the context: value rows are zero
    if (key1 >= ctx) v_reg1 = 0;
  };
  auto stage = [&](int buf) {
    *reinterpret_cast<u32x4*>(&lds_k[buf][k_key * kKRow + 8 * k_chunk]) = k_reg;
    // V^T[d][2*pair .. 2*pair+1] for the four dims of this thread
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = static_cast<uint32_t>(v_reg0 >> (16 * e)) & 0xFFFFu;
      const uint32_t hi = static_cast<uint32_t>(v_reg1 >> (16 * e)) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(&lds_v[buf][(4 * v_quad + e) * kVRow + 2 * v_pair]) =
          lo | (hi << 16);
    }
  };

  float m = -INFINITY;  // running reference (log2 domain) of this lane's query
  float lsum = 0.f;     // this lane's share of the denominator
  f32x4v acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4v{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    stage(buf);
    __syncthreads();
    if (kb + 1 < nkb) fetch(kb + 1);
    if (kb * kKeys <= wave_last) {
      // S^T for this block: 16 keys x 16 queries
      f32x4v sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const f16x8 kop =
            *reinterpret_cast<const f16x8*>(&lds_k[buf][lr * kKRow + 8 * lg + 32 * st]);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[st], sc, 0, 0, 0);
      }
      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb * kKeys + 4 * lg + i;
        sv[i] = key <= pos ? sc[i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      if (__any(mx > m + 8.0f)) {
        const float mn = fmaxf(m, mx);
        const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= alpha;
        m = mn;
      }
      f16x4 pop;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16 p = static_cast<f16>(sv[i] == -INFINITY ? 0.f : fast_exp2(sv[i] - m));
        pop[i] = p;
        lsum += static_cast<float>(p);
      }
      // O^T += V^T . P^T, 16 head dims per product
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x4 vop = *reinterpret_cast<const f16x4*>(&lds_v[buf][(16 * j + lr) * kVRow + 4 * lg]);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop, pop, acc[j], 0, 0, 0);
      }
    }
  }

  // denominator of this lane's query: sum over the four lane groups
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  if (q >= n) return;
  const float inv = 1.f / lsum;
  f16* op = static_cast<f16*>(a.out) + (static_cast<int64_t>(q_first + q) * a.num_heads + h) * kD;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = static_cast<f16>(acc[j][i] * inv);
    *reinterpret_cast<f16x4*>(op + 16 * j + 4 * lg) = o;
  }
}

hipError_t launch_tile(const TileArgs& a, int head_dim, int block_size, int max_query_len,
                       hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int tiles = (max_query_len + kTileQ - 1) / kTileQ;
  dim3 grid(a.num_heads, tiles, a.num_seqs);
  switch (block_size) {
    case 8: hipLaunchKernelGGL(tile_attention_kernel<8>, grid, dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL(tile_attention_kernel<16>, grid, dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL(tile_attention_kernel<32>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
