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
//   * the workgroup stages each step's K and V rows into LDS row-major
//     ([key][dim], padded rows) in a ring of three buffers: while a step's
//     values are consumed, the next step's keys are already in LDS and the
//     step after that is being written, so one barrier per step suffices; the
//     global loads for a step are issued a whole step before they are staged.
//     Each wave stages 8 consecutive rows of a step, which lie in one block
//     (block sizes are multiples of 8), so its block id is a scalar load and
//     every pool address is a scalar block base plus a fixed per-lane offset;
//   * LDS pointers stay in the LDS address space and each step's base is
//     formed once, so every LDS access of a step is that base plus an
//     immediate offset (no per-access address arithmetic);
//   * the loop is software-pipelined: the scores of step i+1,
//     S^T = K . Q^T (four v_mfma_f32_16x16x32_f16 per 16-key subtile and query
//     tile over head_dim 128), are issued in the same block as the
//     exponentials of step i, so the matrix cores and the vector ALU work on
//     independent data.  Lane (g, r) = (l/16, l%16) holds S^T[key 4g+i][query r];
//   * causal masking by absolute key position, applied only on steps that
//     reach a wave's first query position; online softmax with scores kept in
//     raw units and the scale folded into one FMA, p = 2^(s*c - m*c) with
//     c = log2(e)/sqrt(d), so masked scores (-inf) give p = 0 directly.  The
//     running reference m of a query moves only when one of its scores passes
//     it by 2^8 in p: each lane checks its own scores and only a wave vote
//     that finds such a score runs the cross-lane maximum and the rescale;
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
// this file).  Values of keys at or past the context length are zeroed when
// staged (those pool slots may hold anything); keys past a query's position
// are masked.  Waves whose queries all lie past the chunk's end only stage.
//
// Key splits (a compile-time variant): a launch with too few tiles to fill the
// chip gives each tile's key steps to several workgroups, each of which writes
// per-query partials (unnormalised output rows, max and sum) to the workspace;
// tile_merge_kernel combines them with the same online-softmax rule the decode
// merge uses [P2 "PagedAttentionの仕組み", online softmax remark].

#include <math.h>

#include <algorithm>

#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

constexpr int kTileQ = 128;       // queries per workgroup (4 waves x 2 column tiles)
constexpr int kStep = 32;         // keys per step
constexpr int kBufs = 3;          // LDS ring: values of step i, keys of i+1, staging of i+2

// Head-dim dependent geometry (head_dim 64 or 128).
template <int D>
struct TileGeom {
  static constexpr int kSt = D / 32;   // score products per 16-key subtile (32 dims each)
  static constexpr int kJ = D / 16;    // value products per 32-key group (16 dims each)
  // LDS row strides (halves): D + 16, i.e. 288 B for D = 128, on which the 16-byte K operand
  // reads run at the full LDS rate (272 B measured half rate) and the transposing V reads too
  static constexpr int kKRow = D + 16;
  static constexpr int kVRow = D + 16;
  static constexpr int kKBuf = kStep * kKRow;
  static constexpr int kVBuf = kStep * kVRow;
  static constexpr int kChunks = D / 8;                // 16-byte chunks per head row
  static constexpr int kRowsPerLoad = 64 / kChunks;    // rows of one wave load: 4 or 8
  static constexpr int kLoads = 8 / kRowsPerLoad;      // loads per wave, step and matrix: 2 or 1
  static constexpr float kSqrtD = D == 128 ? 11.313708498984761f : 8.0f;
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
};

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __fp16 lds_f16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));

// LDS pointers are kept in the LDS address space, so constant offsets fold into the
// instructions' offset fields.
typedef __attribute__((address_space(3))) f16 lf16;
typedef __attribute__((address_space(3))) f16x8 lf16x8;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) lds_f16x4 llds_f16x4;

// Transposing 8-byte LDS read (see the lane mapping above).
__device__ __forceinline__ f16x4 lds_read_tr(const lf16* p) {
  const lds_f16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((llds_f16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// The per-step LDS base, computed once and hidden from reassociation, so every read of the
// step is that base plus an immediate offset.
__device__ __forceinline__ const lf16* opaque(const lf16* p) {
  asm("" : "+v"(p));
  return p;
}

__device__ __forceinline__ f32x4v mfma16(const f16x8& a, const f16x8& b, const f32x4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Workgroups a tile of `steps` key steps is split over (the tile and merge kernels agree).
__device__ __forceinline__ int tile_splits(const TileArgs& a, int steps) {
  if (a.split_steps <= 0 || steps <= a.split_steps) return 1;
  const int ns = (steps + a.split_steps - 1) / a.split_steps;
  return ns < a.splits_max ? ns : a.splits_max;
}

// Tuning of the key splits: split when a launch has fewer than kSplitTargetWgs tile
// workgroups, into about kSplitTargetWgs / workgroups splits of at least kMinSplitSteps
// steps.  512 = one round of the chip (two tile workgroups per CU): measured on the mixed
// chunk + decode batch at 32/16/8/4 heads, splitting pays only below it (4 heads: 94 vs
// 134 us, 8 heads: 151 vs 167 us); at 16 heads (512 workgroups) splitting into 2 costs 25%
// and at 32 heads into 2-4 costs 25-30% (partial writes, merge, re-staged keys).
constexpr int64_t kSplitTargetWgs = 512;
constexpr int kMinSplitSteps = 16;

}  // namespace

// two waves per SIMD: the register budget of 32 queries per wave
template <int D, int BS, bool kWindow, bool kAlibi, bool kSplit>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void tile_attention_kernel(TileArgs a) {
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  using G = TileGeom<D>;
  constexpr int kD = D;
  constexpr int kKRow = G::kKRow, kVRow = G::kVRow, kKBuf = G::kKBuf, kVBuf = G::kVBuf;
  constexpr int kTab = kStep / BS;  // blocks spanned by one step
  __shared__ __attribute__((aligned(16))) f16 lds_k_[kBufs * kKBuf];
  __shared__ __attribute__((aligned(16))) f16 lds_v_[kBufs * kVBuf];
  lf16* const lds_k = (lf16*)(lds_k_);
  lf16* const lds_v = (lf16*)(lds_v_);

  // head fastest, then (query tile, key split) with the last tiles, which see the most keys,
  // first, then sequence
  const int h = blockIdx.x;
  const int splits_max = kSplit ? a.splits_max : 1;
  const int tile = static_cast<int>(gridDim.y) / splits_max - 1 -
                   static_cast<int>(blockIdx.y) / splits_max;
  const int split = kSplit ? static_cast<int>(blockIdx.y) % splits_max : 0;
  const int s = blockIdx.z;
  const int t = threadIdx.x;
  const int w = t >> 6;  // wave index
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
  // last key any query of the workgroup / of this wave needs (-1: the wave has no query)
  const int wg_last = ctx - n + min(q0 + kTileQ - 1, n - 1);
  const int wave_last = q0 + 32 * w < n ? ctx - n + min(q0 + 32 * w + 31, n - 1) : -1;
  const int nsteps = wg_last / kStep + 1;
  // first query position of this wave: steps ending at or before it need no mask
  const int wave_first_pos = ctx - n + q0 + 32 * w;
  // Sliding window W > 0: the query at position p sees keys p-W+1 .. p.  The workgroup starts
  // at the step holding its first query's window start (older keys are never fetched for
  // use); a wave computes only the steps from its own first query's window start to its last
  // query.  Without a window every wave starts at step 0.
  const int W = kWindow ? a.window : 0;  // compile-time 0 without a window
  const int wg_key_lo = W > 0 ? max(0, ctx - n + q0 - W + 1) : 0;
  const int step_lo = wg_key_lo / kStep;
  // This workgroup's steps: the whole range, or one split of it (the last split takes the rest).
  // Without splits (compile time) the range is the tile's own and the loop compiles as such.
  const int nsplit = kSplit ? tile_splits(a, nsteps - step_lo) : 1;
  if (split >= nsplit) return;
  const int first_step = kSplit ? step_lo + split * a.split_steps : step_lo;
  const int end_step = !kSplit || split == nsplit - 1 ? nsteps : first_step + a.split_steps;
  const int wave_hi_step = wave_last >= 0 ? wave_last / kStep : -1;
  const int wave_lo_step = W > 0 ? max(0, wave_first_pos - W + 1) / kStep : 0;
  // ALiBi: slope_h * (j - p) is added to q.k_j / sqrt(d); in the raw units of the scores here
  // (q.k) that is slope_h * sqrt(d) * (j - p).
  const float slope_sd = kAlibi ? a.alibi[h] * G::kSqrtD : 0.f;

  // Q^T operands: lane (lg, lr) holds dims 8*lg + 32*st .. +7 of its query, st < D/32
  f16x8 qop[2][G::kSt];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const f16* qp = static_cast<const f16*>(a.q) +
                    (static_cast<int64_t>(q_first + min(q[qt], n - 1)) * a.num_heads + h) * kD;
#pragma unroll
    for (int st = 0; st < G::kSt; ++st) {
      u32x4 v = ld16(qp + 8 * lg + 32 * st);
      if (q[qt] >= n) v = u32x4{0, 0, 0, 0};
      qop[qt][st] = __builtin_bit_cast(f16x8, v);
    }
  }

  const int64_t row_stride = static_cast<int64_t>(a.num_heads) * kD;
  const f16* kpool = static_cast<const f16*>(a.k_pool) + static_cast<int64_t>(h) * kD;
  const f16* vpool = static_cast<const f16*>(a.v_pool) + static_cast<int64_t>(h) * kD;
  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  const int last_blk = (ctx - 1) / BS;

  // Staging: wave ws stages the 8 rows 8*ws .. 8*ws+7 of each step: load r covers rows
  // 8*ws + R*r + l/C (R = 64/C rows, C = D/8 16-byte chunks per row), chunk l%C.  The 8 rows
  // lie in one block (block sizes are multiples of 8), so the block id is wave-uniform and the
  // pool address is a scalar block base plus a fixed per-lane offset.
  constexpr int kC = G::kChunks, kR = G::kRowsPerLoad, kL = G::kLoads;
  const int ws = __builtin_amdgcn_readfirstlane(t >> 6);
  const int srow = 8 * ws + l / kC;  // this lane's first staged row
  const int schunk = l % kC;
  const int64_t block_elems = static_cast<int64_t>(BS) * row_stride;
  uint32_t toff[kL];
#pragma unroll
  for (int r = 0; r < kL; ++r)
    toff[r] = static_cast<uint32_t>((((srow + kR * r) % BS) * row_stride + 8 * schunk) * 2);
  const char* kpool_b = reinterpret_cast<const char*>(kpool);
  const char* vpool_b = reinterpret_cast<const char*>(vpool);
  u32x4 k_reg[kL], v_reg[kL];
  // block id of this wave's rows in `step` (clamped to the last used block; invalid ids
  // read block 0, so every address stays inside the pool)
  const uint32_t nblk32 =
      static_cast<uint32_t>(a.num_blocks < INT32_MAX ? a.num_blocks : INT32_MAX);
  auto block_of = [&](int step) {
    const int idx = min(step * kTab + (8 * ws) / BS, last_blk);
    const int b = btrow[idx];
    return static_cast<uint32_t>(b) < nblk32 ? b : 0;
  };
  auto fetch = [&](int step, int blk) {
    const int64_t boff = static_cast<int64_t>(blk) * block_elems * 2;
    const char* kb = kpool_b + boff;
    const char* vb = vpool_b + boff;
#pragma unroll
    for (int r = 0; r < kL; ++r) {
      k_reg[r] = ld16(kb + toff[r]);
      v_reg[r] = ld16(vb + toff[r]);
    }
    if (step * kStep + kStep > ctx) {  // the step holding the context's end (wave-uniform)
#pragma unroll
      for (int r = 0; r < kL; ++r)
        if (step * kStep + srow + kR * r >= ctx) v_reg[r] = u32x4{0, 0, 0, 0};
    }
    if (step * kStep < wg_key_lo) {  // the step holding the window's start: older slots may
#pragma unroll                       // hold anything (their blocks may even be released)
      for (int r = 0; r < kL; ++r)
        if (step * kStep + srow + kR * r < wg_key_lo) v_reg[r] = u32x4{0, 0, 0, 0};
    }
  };
  const int kst_off = srow * kKRow + 8 * schunk;
  const int vst_off = srow * kVRow + 8 * schunk;
  auto stage = [&](int buf) {
    lf16* kd = lds_k + buf * kKBuf + kst_off;
    lf16* vd = lds_v + buf * kVBuf + vst_off;
#pragma unroll
    for (int r = 0; r < kL; ++r) {
      *(lu32x4*)(kd + kR * r * kKRow) = k_reg[r];
      *(lu32x4*)(vd + kR * r * kVRow) = v_reg[r];
    }
  };

  // Scores stay in raw units (q.k); c = log2(e)/sqrt(d) is folded into one FMA with the
  // running reference: p = 2^(s*c - m*c).  Masked scores are -inf and give p = 0.
  const float c = a.scale_log2;
  const float tau = 8.0f / c;           // reference margin, 2^8 in p
  float m[2] = {-INFINITY, -INFINITY};  // running reference (raw units) per query tile
  float mc[2] = {0.f, 0.f};             // m*c, 0 while m is still -inf
  f32x4v acc[2][G::kJ];
  f32x4v den[2];                        // O^T row of a ones "dimension": sum of P (row 0)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    den[qt] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < G::kJ; ++j) acc[qt][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  }
  // V^T operand of the ones row: lane (g, 0) holds eight ones, every other lane zeros
  f16x8 ones_op;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones_op[e] = static_cast<f16>(lr == 0 ? 1.f : 0.f);

  const lf16* const kbase = lds_k + lr * kKRow + 8 * lg;
  const lf16* const vbase = lds_v + (4 * lg + (lr >> 2)) * kVRow + 4 * (lr & 3);

  // S^T of the step at key `base` for both query tiles: sc[qt][sub] holds keys
  // base + 16*sub + 4*lg + i.  With ALiBi the accumulators start at the bias, so the products
  // add q.k onto it.
  // The K^T operands of a step: lane (g, r) holds dims 8g + 32st .. +7 of key r (+16 sub).
  auto load_k = [&](int buf, f16x8 (&kop)[2][G::kSt]) {
    const lf16* kb = opaque(kbase + buf * kKBuf);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int st = 0; st < G::kSt; ++st)
        kop[sub][st] = *(const lf16x8*)(kb + (16 * sub) * kKRow + 32 * st);
  };
  auto scores_of = [&](const f16x8 (&kop)[2][G::kSt], int base, f32x4v (&sc)[2][2]) {
    if constexpr (kAlibi) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float fd = static_cast<float>(base + 4 * lg - pos[qt]);  // j - p for sub = i = 0
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[qt][sub][i] = slope_sd * (fd + static_cast<float>(16 * sub + i));
      }
    } else {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) sc[qt][sub] = f32x4v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int st = 0; st < G::kSt; ++st)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          sc[qt][sub] = mfma16(kop[sub][st], qop[qt][st], sc[qt][sub]);
  };
  auto scores = [&](int buf, int base, f32x4v (&sc)[2][2]) {
    f16x8 kop[2][G::kSt];
    load_k(buf, kop);
    scores_of(kop, base, sc);
  };

  // Causal (and window) mask and the reference update for the scores of the step at `base`.
  auto prepare = [&](int base, f32x4v (&sc)[2][2]) {
    // masking runs only on steps that reach this wave's diagonal or hold some query's window
    // start
    if (base + kStep - 1 > wave_first_pos || (W > 0 && base < wave_last - W + 1)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int lo = W > 0 ? pos[qt] - W + 1 : INT32_MIN;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = base + 16 * sub + 4 * lg + i;
            if (key > pos[qt] || key < lo) sc[qt][sub][i] = -INFINITY;
          }
      }
    }
    float lmax[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float v = fmaxf(fmaxf(sc[qt][0][0], sc[qt][0][1]), sc[qt][0][2]);
      v = fmaxf(fmaxf(v, sc[qt][0][3]), sc[qt][1][0]);
      v = fmaxf(fmaxf(v, sc[qt][1][1]), sc[qt][1][2]);
      lmax[qt] = fmaxf(v, sc[qt][1][3]);
    }
    if (__any(lmax[0] > m[0] + tau || lmax[1] > m[1] + tau)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float mx = lmax[qt];
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const float mn = fmaxf(m[qt], mx);
        const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2((m[qt] - mn) * c);
        den[qt] *= alpha;
#pragma unroll
        for (int j = 0; j < G::kJ; ++j) acc[qt][j] *= alpha;
        m[qt] = mn;
        mc[qt] = (mn == -INFINITY) ? 0.f : mn * c;
      }
    }
  };

  // P^T operands (keys 4g+i then 16+4g+i) and O^T += V^T . P^T for the step in `buf`.
  auto exps = [&](const f32x4v (&sc)[2][2], f16x8 (&pop)[2]) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pop[qt][4 * sub + i] = static_cast<f16>(fast_exp2(fmaf(sc[qt][sub][i], c, -mc[qt])));
  };
  auto values = [&](int buf, const f16x8 (&pop)[2]) {
    const lf16* vrow0 = opaque(vbase + buf * kVBuf);
    const lf16* vrow1 = vrow0 + 16 * kVRow;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) den[qt] = mfma16(ones_op, pop[qt], den[qt]);
#pragma unroll
    for (int j = 0; j < G::kJ; ++j) {
      const f16x4 va = lds_read_tr(vrow0 + 16 * j);
      const f16x4 vb = lds_read_tr(vrow1 + 16 * j);
      const f16x8 vop = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) acc[qt][j] = mfma16(vop, pop[qt], acc[qt][j]);
    }
  };

  int blk_next;  // block id of this wave's rows in the next step to fetch
  // One pipelined step: values of `step` (scores in `cur`), scores of step+1 into `nxt`.
  // LDS buffers are numbered from the first step of the workgroup.
  auto iteration = [&](int step, f32x4v (&cur)[2][2], f32x4v (&nxt)[2][2]) {
    const int rel = step - first_step;
    const int b_cur = rel % kBufs;
    const int b_nxt = (rel + 1) % kBufs;
    if (step + 2 < end_step) stage((rel + 2) % kBufs);
    if (step + 3 < end_step) {
      fetch(step + 3, blk_next);
      if (step + 4 < end_step) blk_next = block_of(step + 4);
    }
    const int base = step * kStep;
    const bool cur_on = step >= wave_lo_step && step <= wave_hi_step;
    const bool nxt_on = step + 1 >= wave_lo_step && step + 1 <= wave_hi_step;
    if (cur_on && nxt_on) {
      // the next step's K rows have been in LDS since the last barrier: read them before the
      // reference update, so their latency overlaps it instead of stalling the score products
      // (read at their use, the products waited on four LDS round trips per step: 5% slower)
      f16x8 kop[2][G::kSt];
      load_k(b_nxt, kop);
      prepare(base, cur);
      f16x8 pop[2];
      scores_of(kop, base + kStep, nxt);
      exps(cur, pop);
      values(b_cur, pop);
    } else if (cur_on) {
      prepare(base, cur);
      f16x8 pop[2];
      exps(cur, pop);
      values(b_cur, pop);
    } else if (nxt_on) {  // the step before this wave's window: its first scores
      scores(b_nxt, base + kStep, nxt);
    }
    __syncthreads();
  };

  // prologue: the first two steps staged, the third in flight, scores of the first step
  blk_next = block_of(first_step);
  fetch(first_step, blk_next);
  stage(0);
  if (first_step + 1 < end_step) {
    fetch(first_step + 1, block_of(first_step + 1));
    stage(1);
  }
  if (first_step + 2 < end_step) fetch(first_step + 2, block_of(first_step + 2));
  if (first_step + 3 < end_step) blk_next = block_of(first_step + 3);
  __syncthreads();
  f32x4v sa[2][2], sb[2][2];
  if (wave_lo_step <= first_step && first_step <= wave_hi_step)
    scores(0, first_step * kStep, sa);

  int step = first_step;
  for (; step + 1 < end_step; step += 2) {
    iteration(step, sa, sb);
    iteration(step + 1, sb, sa);
  }
  if (step < end_step) iteration(step, sa, sb);

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    // denominator of this lane's query: row 0 of the ones product, held by lane (0, lr)
    const float total = __shfl(den[qt][0], lr, kWave);
    if (q[qt] >= n) continue;
    const int64_t row = static_cast<int64_t>(q_first + q[qt]) * a.num_heads + h;
    if (!kSplit || nsplit == 1) {
      const float inv = 1.f / total;
      f16* op = static_cast<f16*>(a.out) + row * kD;
#pragma unroll
      for (int j = 0; j < G::kJ; ++j) {
        f16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = static_cast<f16>(acc[qt][j][i] * inv);
        *reinterpret_cast<f16x4*>(op + 16 * j + 4 * lg) = o;
      }
    } else {
      // this split's partial: unnormalised O^T rows, (reference m*c, sum) in log2 units;
      // a query with no key in the split has m = -inf and weight 0 in the merge
      const int64_t slot = row * a.num_parts_max + split;
      float* wp = a.ws_acc + slot * kD;
#pragma unroll
      for (int j = 0; j < G::kJ; ++j) *reinterpret_cast<f32x4v*>(wp + 16 * j + 4 * lg) = acc[qt][j];
      if (lg == 0) {
        a.ws_ml[2 * slot] = m[qt] == -INFINITY ? -INFINITY : mc[qt];
        a.ws_ml[2 * slot + 1] = total;
      }
    }
  }
}

// Merge of split tiles: for each query row and head, M = max_p m_p and
// o = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p over the tile's splits (the online-
// softmax merge rule, as for decode partitions).  One workgroup per (head, 8 rows of a tile,
// sequence), 32 lanes per row: the partial loads of different splits are independent, so a
// row's latency is about one load, and the many small workgroups keep enough in flight.
constexpr int kMergeRows = 8;
constexpr int kMergeGroups = kTileQ / kMergeRows;

template <int D>
__global__ __launch_bounds__(256) void tile_merge_kernel(TileArgs a) {
  constexpr int kPer = D / 32;  // dims per lane: 4 or 2
  const int h = blockIdx.x;
  const int tile = static_cast<int>(blockIdx.y) / kMergeGroups;
  const int s = blockIdx.z;
  const int q_first = a.q_start_loc[s];
  const int n = a.q_start_loc[s + 1] - q_first;
  if (n <= 1) return;
  const int q0 = tile * kTileQ;
  const int r = q0 + (static_cast<int>(blockIdx.y) % kMergeGroups) * kMergeRows +
                static_cast<int>(threadIdx.x >> 5);
  if (r >= n) return;
  const int ctx = min(a.context_lens[s], a.max_blocks * a.block_size);
  if (n > ctx || q_first < 0 || q_first + n > a.num_tokens) return;
  // the tile kernel's step range and split count for this tile
  const int wg_last = ctx - n + min(q0 + kTileQ - 1, n - 1);
  const int nsteps = wg_last / kStep + 1;
  const int wg_key_lo = a.window > 0 ? max(0, ctx - n + q0 - a.window + 1) : 0;
  const int nsplit = tile_splits(a, nsteps - wg_key_lo / kStep);
  if (nsplit <= 1) return;
  const int c = threadIdx.x & 31;
  const int64_t row = static_cast<int64_t>(q_first + r) * a.num_heads + h;
  const int64_t slot0 = row * a.num_parts_max;
  const float* ml = a.ws_ml + slot0 * 2;
  float M = -INFINITY;
  for (int p = 0; p < nsplit; ++p) M = fmaxf(M, ml[2 * p]);
  float L = 0.f;
  float o[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) o[i] = 0.f;
  const float* acc = a.ws_acc + slot0 * D + c * kPer;
#pragma unroll 4
  for (int p = 0; p < nsplit; ++p) {
    const float w = fast_exp2(ml[2 * p] - M);
    L = fmaf(w, ml[2 * p + 1], L);
    const float* ap = acc + static_cast<int64_t>(p) * D;
    if constexpr (kPer == 4) {
      const f32x4v v = *reinterpret_cast<const f32x4v*>(ap);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(w, v[i], o[i]);
    } else {
      const float2 v = *reinterpret_cast<const float2*>(ap);
      o[0] = fmaf(w, v.x, o[0]);
      o[1] = fmaf(w, v.y, o[1]);
    }
  }
  const float inv = 1.f / L;
  f16* op = static_cast<f16*>(a.out) + row * D + c * kPer;
#pragma unroll
  for (int i = 0; i < kPer; ++i) op[i] = static_cast<f16>(o[i] * inv);
}

hipError_t launch_tile(const TileArgs& a0, void* workspace, int head_dim, int block_size,
                       int max_query_len, int max_context_len, hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  TileArgs a = a0;
  a.block_size = block_size;
  const int tiles = (max_query_len + kTileQ - 1) / kTileQ;
  // Key splits, when the launch has too few tile workgroups to fill the chip: the chunks hold
  // at least ceil((num_tokens - num_seqs) / kTileQ) tiles (every sequence has one query row
  // outside the count).  Partials use the workspace at its common slot stride.
  a.num_parts_max = workspace_parts(max_context_len);
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = a.ws_acc + static_cast<int64_t>(a.num_tokens) * a.num_heads * a.num_parts_max *
                           head_dim;
  a.split_steps = 0;
  a.splits_max = 1;
  const int max_steps = (max_context_len + kStep - 1) / kStep;
  const int64_t wgs =
      std::max<int64_t>(1, (int64_t{a.num_tokens} - a.num_seqs + kTileQ - 1) / kTileQ) *
      a.num_heads;
  if (workspace != nullptr && a.num_parts_max > 1 && wgs < kSplitTargetWgs) {
    const int want = static_cast<int>((kSplitTargetWgs + wgs - 1) / wgs);
    const int ss = std::max((max_steps + want - 1) / want, kMinSplitSteps);
    const int ns = std::min((max_steps + ss - 1) / ss, a.num_parts_max);
    if (ss < max_steps && ns > 1 && int64_t{tiles} * std::max(ns, kMergeGroups) <= 65535) {
      a.split_steps = ss;
      a.splits_max = ns;
    }
  }
  dim3 grid(a.num_heads, tiles * a.splits_max, a.num_seqs);
  const bool window = a.window > 0;
  const bool alibi = a.alibi != nullptr;
  const bool split = a.splits_max > 1;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a); };
  // (head_dim, block size, window, ALiBi) pick one instantiation
#define PA_TILE_SPLITS(D_, B_, W_, A_)                                             \
  if (split) go(tile_attention_kernel<D_, B_, W_, A_, true>);                      \
  else go(tile_attention_kernel<D_, B_, W_, A_, false>);
#define PA_TILE_VARIANTS(D_, B_)                                                   \
  if (window && alibi) { PA_TILE_SPLITS(D_, B_, true, true) }                      \
  else if (window) { PA_TILE_SPLITS(D_, B_, true, false) }                         \
  else if (alibi) { PA_TILE_SPLITS(D_, B_, false, true) }                          \
  else { PA_TILE_SPLITS(D_, B_, false, false) }
#define PA_TILE_BLOCKS(D_)                                                         \
  switch (block_size) {                                                            \
    case 8: PA_TILE_VARIANTS(D_, 8) break;                                         \
    case 16: PA_TILE_VARIANTS(D_, 16) break;                                       \
    case 32: PA_TILE_VARIANTS(D_, 32) break;                                       \
    default: return hipErrorInvalidValue;                                          \
  }
  if (head_dim == 128) {
    PA_TILE_BLOCKS(128)
  } else {
    PA_TILE_BLOCKS(64)
  }
#undef PA_TILE_BLOCKS
#undef PA_TILE_VARIANTS
#undef PA_TILE_SPLITS
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.splits_max <= 1) return err;
  dim3 grid2(a.num_heads, tiles * kMergeGroups, a.num_seqs);
  if (head_dim == 128)
    hipLaunchKernelGGL(tile_merge_kernel<128>, grid2, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(tile_merge_kernel<64>, grid2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
