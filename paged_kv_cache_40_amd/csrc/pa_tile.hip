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
// One workgroup = 4 waves = 128 consecutive queries of one (sequence, head);
// wave w owns queries q0+32w .. q0+32w+31 as two 16-query column tiles, so
// every operand it reads from LDS feeds two matrix products.  Keys are
// processed 32 per step:
//   * the workgroup stages the step's K and V rows into LDS row-major
//     ([key][dim], padded rows), double-buffered with one barrier per step,
//     while the next step's rows are already in flight to registers;
//   * S^T = K . Q^T per 16-key subtile and query tile: four
//     v_mfma_f32_16x16x32_f16 over head_dim 128; lane (g, r) = (l/16, l%16)
//     holds S^T[key 4g+i][query r], so every per-query quantity lives in the
//     lanes of one column;
//   * causal masking by absolute key position, applied only on steps that
//     reach a query's own position; online softmax with scores kept in raw
//     units and the scale folded into one FMA, p = 2^(s*c - m*c) with
//     c = log2(e)/sqrt(d), so masked scores (-inf) give p = 0 directly; the
//     running reference m moves only when a score passes it by 2^8 in p;
//     P^T rounded to fp16;
//   * O^T += V^T . P^T with v_mfma_f32_16x16x32_f16 over the step's 32 keys.
//     The V^T operand comes straight from the row-major V rows through the
//     transposing LDS read ds_read_b64_tr_b16: within each 16-lane group,
//     lane L receives element L%4 of the 8-byte chunks addressed by lanes
//     4i + L/4 (i = 0..3), so when lane j addresses V[k0 + j/4][d0 + 4(j%4)]
//     lane L gets keys k0..k0+3 of head dim d0+L.  Lane group g takes keys
//     4g..4g+3 and 16+4g..16+4g+3 — the keys its own P^T registers hold — so
//     both operands index keys in the same (permuted) order, which leaves the
//     product over keys unchanged;
//   * the softmax denominator is one more product of the same kind against a
//     constant operand whose row 0 is all ones, so it sums exactly the
//     fp16-rounded P values the value product uses, on the matrix cores.
// Accumulators live in VGPRs (the build passes -amdgpu-mfma-vgpr-form for
// this file); the last query tiles, which see the most keys, are dispatched
// first.
// Values of keys at or past the context length are zeroed when staged (those
// pool slots may hold anything), keys past a query's position are masked.

#include <math.h>

#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

constexpr int kTileQ = 128;       // queries per workgroup (4 waves x 2 column tiles)
#ifndef PA_TILE_STEP
#define PA_TILE_STEP 32
#endif
constexpr int kStep = PA_TILE_STEP;  // keys per step (a multiple of 32)
constexpr int kGroups = kStep / 32;  // 32-key groups per step
static_assert(kStep % 32 == 0, "steps hold whole 32-key groups");
constexpr int kD = 128;           // head dim of the tile path
constexpr int kKRow = kD + 8;     // K row stride in LDS (halves): 272 B, 16-byte reads spread banks
constexpr int kVRow = kD + 16;    // V row stride in LDS (halves): 288 B, transposing reads spread banks
constexpr int kKBuf = kStep * kKRow;
constexpr int kVBuf = kStep * kVRow;

#ifndef PA_TILE_NT_LOADS
#define PA_TILE_NT_LOADS 0  // K/V rows are re-read by every query tile of a head: keep them cached
#endif
#ifndef PA_TILE_BULK_LDS
#define PA_TILE_BULK_LDS 0  // 1: read all LDS operands of a step before its products
#endif
#ifndef PA_TILE_HEAVY_FIRST
#define PA_TILE_HEAVY_FIRST 1  // dispatch the last query tiles (most keys) first
#endif

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __fp16 lds_f16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));

// Transposing 8-byte LDS read (see the lane mapping above).
__device__ __forceinline__ f16x4 lds_read_tr(const f16* p) {
  typedef __attribute__((address_space(3))) lds_f16x4* lptr;
  const lds_f16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lptr)(p));
  return __builtin_bit_cast(f16x4, v);
}

}  // namespace

#ifndef PA_TILE_WAVES_PER_EU
#define PA_TILE_WAVES_PER_EU 2  // 3 per SIMD spills registers and runs slower
#endif
#if PA_TILE_WAVES_PER_EU > 0
#define PA_TILE_OCCUPANCY __attribute__((amdgpu_waves_per_eu(PA_TILE_WAVES_PER_EU)))
#else
#define PA_TILE_OCCUPANCY
#endif

template <int BS>
__global__ __launch_bounds__(256) PA_TILE_OCCUPANCY void tile_attention_kernel(TileArgs a) {
  __shared__ __attribute__((aligned(16))) f16 lds_k[2][kKBuf];
  __shared__ __attribute__((aligned(16))) f16 lds_v[2][kVBuf];

  const int h = blockIdx.x;
#if PA_TILE_HEAVY_FIRST
  const int tile = static_cast<int>(gridDim.y) - 1 - static_cast<int>(blockIdx.y);
#else
  const int tile = blockIdx.y;
#endif
  const int s = blockIdx.z;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int l = t & 63;
  const int lg = l >> 4;  // lane group 0..3
  const int lr = l & 15;  // column within a 16-query tile

  const int q_first = a.q_start_loc[s];
  const int n = a.q_start_loc[s + 1] - q_first;
  if (n <= 1) return;  // single-query sequences run the decode path
  const int q0 = tile * kTileQ;
  if (q0 >= n) return;
  const int ctx = min(a.context_lens[s], a.max_blocks * BS);
  if (n > ctx || q_first < 0 || q_first + n > a.num_tokens) return;

  // this lane's two queries and their absolute positions (-1 = no query: fully masked)
  int q[2], pos[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    q[qt] = q0 + 32 * w + 16 * qt + lr;
    pos[qt] = q[qt] < n ? ctx - n + q[qt] : -1;
  }
  // last key any query of the workgroup / of this wave needs
  const int wg_last = ctx - n + min(q0 + kTileQ - 1, n - 1);
  const int wave_last = ctx - n + min(q0 + 32 * w + 31, n - 1);
  const int nsteps = wg_last / kStep + 1;

  // Q^T operands: lane (lg, lr) holds dims 8*lg + 32*st .. +7 of its query, st = 0..3
  f16x8 qop[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const f16* qp = static_cast<const f16*>(a.q) +
                    (static_cast<int64_t>(q_first + min(q[qt], n - 1)) * a.num_heads + h) * kD;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4 v = ld16(qp + 8 * lg + 32 * st);
      if (q[qt] >= n) v = u32x4{0, 0, 0, 0};
      qop[qt][st] = __builtin_bit_cast(f16x8, v);
    }
  }

  const int64_t row_stride = static_cast<int64_t>(a.num_heads) * kD;
  const f16* kpool = static_cast<const f16*>(a.k_pool) + static_cast<int64_t>(h) * kD;
  const f16* vpool = static_cast<const f16*>(a.v_pool) + static_cast<int64_t>(h) * kD;
  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;

  // staging: thread -> rows 16r + t/16 (r = 0..kStep/16-1) of the step, 16-byte chunk t%16
  constexpr int kRows = kStep / 16;
  const int st_row = t >> 4, st_chunk = t & 15;
  u32x4 k_reg[kRows], v_reg[kRows];
  // block ids of the rows this thread stages, looked up one step ahead of their use
  int blk_next[kRows];
  auto lookup = [&](int step) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int key = min(step * kStep + 16 * r + st_row, ctx - 1);
      const int b = btrow[key / BS];
      blk_next[r] = (b >= 0 && b < a.num_blocks) ? b : 0;
    }
  };
  auto fetch = [&](int step) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int key = step * kStep + 16 * r + st_row;
      const int64_t row =
          (static_cast<int64_t>(blk_next[r]) * BS + min(key, ctx - 1) % BS) * row_stride;
#if PA_TILE_NT_LOADS
      k_reg[r] = ld16_stream(kpool + row + 8 * st_chunk);
      const u32x4 v = ld16_stream(vpool + row + 8 * st_chunk);
#else
      k_reg[r] = ld16(kpool + row + 8 * st_chunk);
      const u32x4 v = ld16(vpool + row + 8 * st_chunk);
#endif
      v_reg[r] = key < ctx ? v : u32x4{0, 0, 0, 0};  // keys past the context: zero values
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      *reinterpret_cast<u32x4*>(&lds_k[buf][(16 * r + st_row) * kKRow + 8 * st_chunk]) = k_reg[r];
      *reinterpret_cast<u32x4*>(&lds_v[buf][(16 * r + st_row) * kVRow + 8 * st_chunk]) = v_reg[r];
    }
  };

  // Scores stay in raw units (q.k); c = log2(e)/sqrt(d) is folded into one FMA with the
  // running reference: p = 2^(s*c - m*c).  Masked scores are -inf and give p = 0.
  const float c = a.scale_log2;
  const float tau = 8.0f / c;           // reference margin, 2^8 in p
  float m[2] = {-INFINITY, -INFINITY};  // running reference (raw units) per query tile
  float mc[2] = {0.f, 0.f};             // m*c, 0 while m is still -inf
  f32x4v acc[2][8];
  f32x4v den[2];                        // O^T row of a ones "dimension": sum of P (row 0)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    den[qt] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[qt][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  }
  // V^T operand of the ones row: lane (g, 0) holds eight ones, every other lane zeros
  f16x8 ones_op;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones_op[e] = static_cast<f16>(lr == 0 ? 1.f : 0.f);
  // first query position of this wave: steps ending at or before it need no mask
  const int wave_first_pos = ctx - n + q0 + 32 * w;

  lookup(0);
  fetch(0);
  if (nsteps > 1) lookup(1);
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    stage(buf);
    __syncthreads();
    if (step + 1 < nsteps) {
      fetch(step + 1);
      if (step + 2 < nsteps) lookup(step + 2);
    }
    const int base = step * kStep;
    if (base > wave_last) continue;  // every query of this wave precedes the step

    // S^T for the step's 16-key subtiles x two query tiles
    constexpr int kSub = 2 * kGroups;
    f32x4v sc[2][kSub];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) sc[qt][sub] = f32x4v{0.f, 0.f, 0.f, 0.f};
#if PA_TILE_BULK_LDS
    f16x8 kops[kSub][4];
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kops[sub][st] = *reinterpret_cast<const f16x8*>(
            &lds_k[buf][(16 * sub + lr) * kKRow + 8 * lg + 32 * st]);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          sc[qt][sub] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(kops[sub][st], qop[qt][st], sc[qt][sub], 0, 0, 0);
#else
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const f16x8 kop = *reinterpret_cast<const f16x8*>(
            &lds_k[buf][(16 * sub + lr) * kKRow + 8 * lg + 32 * st]);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          sc[qt][sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[qt][st], sc[qt][sub], 0, 0, 0);
      }
#endif
    // mask keys past each query's position (only on steps that reach the diagonal)
    if (base + kStep - 1 > wave_first_pos) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (base + 16 * sub + 4 * lg + i > pos[qt]) sc[qt][sub][i] = -INFINITY;
    }
    float mx[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      mx[qt] = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx[qt] = fmaxf(mx[qt], sc[qt][sub][i]);
      mx[qt] = fmaxf(mx[qt], shfl_xor_f(mx[qt], 16));
      mx[qt] = fmaxf(mx[qt], shfl_xor_f(mx[qt], 32));
    }
    if (__any(mx[0] > m[0] + tau || mx[1] > m[1] + tau)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float mn = fmaxf(m[qt], mx[qt]);
        const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2((m[qt] - mn) * c);
        den[qt] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[qt][j] *= alpha;
        m[qt] = mn;
        mc[qt] = (mn == -INFINITY) ? 0.f : mn * c;
      }
    }
    // P^T operands per (query tile, 32-key group G): keys 32G+4g+i then 32G+16+4g+i
    f16x8 pop[2][kGroups];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pop[qt][sub >> 1][4 * (sub & 1) + i] =
              static_cast<f16>(fast_exp2(fmaf(sc[qt][sub][i], c, -mc[qt])));
    // O^T += V^T . P^T, 16 head dims x 32 keys per product; the ones row sums P
#pragma unroll
    for (int G = 0; G < kGroups; ++G) {
      const f16* vrow0 = &lds_v[buf][(32 * G + 4 * lg + (lr >> 2)) * kVRow + 4 * (lr & 3)];
      const f16* vrow1 = vrow0 + 16 * kVRow;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        den[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones_op, pop[qt][G], den[qt], 0, 0, 0);
#if PA_TILE_BULK_LDS
      f16x8 vops[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x4 va = lds_read_tr(vrow0 + 16 * j);
        const f16x4 vb = lds_read_tr(vrow1 + 16 * j);
        vops[j] = f16x8{va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          acc[qt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vops[j], pop[qt][G], acc[qt][j], 0, 0, 0);
#else
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x4 va = lds_read_tr(vrow0 + 16 * j);
        const f16x4 vb = lds_read_tr(vrow1 + 16 * j);
        const f16x8 vop = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          acc[qt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[qt][G], acc[qt][j], 0, 0, 0);
      }
#endif
    }
  }

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    // denominator of this lane's query: row 0 of the ones product, held by lane (0, lr)
    const float total = __shfl(den[qt][0], lr, kWave);
    if (q[qt] >= n) continue;
    const float inv = 1.f / total;
    f16* op = static_cast<f16*>(a.out) +
              (static_cast<int64_t>(q_first + q[qt]) * a.num_heads + h) * kD;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = static_cast<f16>(acc[qt][j][i] * inv);
      *reinterpret_cast<f16x4*>(op + 16 * j + 4 * lg) = o;
    }
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
