// Paged decode attention for gfx950: one query per (sequence, head), keys and
// values fetched block by block through the block table.
//
// Sources: P1 = "Efficient Memory Management for Large Language Model Serving
// with PagedAttention" (urban-dandelion.tistory.com/4); P2 = "SOSP 2023論文解説:
// vLLM — PagedAttentionによるKVキャッシュメモリ管理の革新".
//
// What is computed [P1 sec. 4, attention equation; P2 "PagedAttentionの仕組み"]:
//   o = sum_j softmax_j(q . k_j / sqrt(d)) v_j over the sequence's tokens j,
// with token j's rows at block_tables[s][j / B], slot j % B [P1 sec. 4, the
// addressing sentence; Fig. 7].  The sum is split into context partitions
// whose partial results are merged exactly with the online-softmax rule
// [P2 "PagedAttentionの仕組み", online softmax remark]:
//   m = max_p m_p;  o = sum_p 2^(m_p - m) acc_p / sum_p 2^(m_p - m) l_p.
//
// Pass 1: one wave per (sequence, head, partition of P tokens); the waves of kHeadsPerWg
//   heads of one (sequence, partition) form a workgroup when that divides the head count.
//   * Lane layout: lane = 8*g + c.  Each load instruction reads one 128-byte
//     cache line of 8 consecutive tokens' head rows: lane (g, c) takes the
//     16 bytes at column c of token g's line.  A head row of kRow bytes spans
//     kCpt = kRow/128 lines, so a lane holds kCpt 16-byte chunks per token
//     and covers kR = 4/kCpt tokens per iteration (four K loads and four V
//     loads per lane per iteration, 8*kR tokens).  A trip covers kU
//     iterations and issues all of its K and V loads before using any.
//   * The 8 tokens of one load share a block (block sizes are multiples of
//     8), so each block id is a wave-uniform readlane from the partition's
//     table entries, loaded once (one per lane).
//   * q.k: v_dot2_f32_f16 (fp16) or fma (fp32) over the lane's chunks, then a
//     DPP sum over the token's 8 lanes (quad_perm xor 1, xor 2, half-row mirror).
//   * Softmax runs in the log2 domain (scores pre-multiplied by log2(e)/sqrt(d),
//     v_exp_f32).  Each lane keeps (m, l, acc) for its own token positions;
//     the running reference m only moves when some lane sees a score more
//     than kTau above it (a wave vote), since any reference gives the same
//     ratio and exponents stay below 2^kTau.
//   * At the end the 8 token groups are merged (xor 8, 16, 32) to one
//     (m, l, acc[d]); a sequence with a single partition writes the
//     normalised output directly.
// Pass 2: one 64-lane workgroup per (sequence, head) with more than one
//   partition merges the partials and writes out.
//
// All pool offsets are 64-bit.  Context lengths are clamped to the table
// width and to the host bound (a sequence with no tokens is skipped), and
// block ids outside [0, num_blocks) are replaced by block 0, so malformed
// device data cannot address memory outside the pools or the workspace.

#include <math.h>
#include <algorithm>

#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

// K/V loads.  Unshared batches stream (each row is read once: the non-temporal hint keeps it
// from displacing useful lines); batches whose neighbouring sequences share blocks keep the
// rows cached so the sharers find them in L2.
template <bool kShared>
__device__ __forceinline__ u32x4 ld_kv(const void* p) {
  if constexpr (!kShared) return ld16_stream(p);
  return ld16(p);
}

template <typename T, int D, int BS, int P, int kTripU = 1>
struct DecodeCfg {
  static constexpr int kElt = sizeof(T);
  static constexpr int kRow = D * kElt;        // bytes of one head's row of one token
  static constexpr int kCpt = kRow / 128;      // 16-byte chunks per lane per token
  static constexpr int kR = 4 / kCpt;          // tokens per lane per iteration
  static constexpr int kTpi = 8 * kR;          // tokens per iteration
  static constexpr int kEpc = 16 / kElt;       // elements per 16-byte chunk
  static constexpr int kEpl = kCpt * kEpc;     // elements (head dims) per lane
  static constexpr int kU = kTripU;             // iterations per trip
  static constexpr int kG = kU * kR;           // token groups per lane per trip
  static constexpr int kTrip = kU * kTpi;      // tokens per trip
  static constexpr int kBlocks = P / BS;       // table entries per partition
  static constexpr int kTabRegs = (kBlocks + kWave - 1) / kWave;  // table entries per lane
  static constexpr int kAlign = kTrip > BS ? kTrip : BS;  // partition starts are multiples
  static_assert(kCpt >= 1 && kCpt <= 4 && 4 % kCpt == 0, "head row must be 1, 2 or 4 lines");
  static_assert(BS % 8 == 0, "a load's 8 tokens must share a block");
  static_assert(P % kTrip == 0 && P % BS == 0, "partition must hold whole trips and blocks");
  static_assert(kTabRegs <= 2, "at most two table entries per lane");
};

constexpr float kTau = 8.0f;  // log2 headroom before the running reference moves

// Heads per workgroup, chosen per launch: kHeadsPerWg when it divides the head count, else
// one.  A partial last group would leave wave slots empty in every (sequence, partition):
// 5 heads in groups of 4 fill 5 of 8 slots, and one head per workgroup runs such batches
// 1.3-1.6x faster, while with 40 heads groups of 4 beat single heads by 4%.
constexpr int kHeadsPerWg = 4;
constexpr int kXcds = 8;        // accelerator complex dies of an MI355X
constexpr int kXcdChunk = 128;  // work units per run on one XCD (shared-block mode)

template <typename T, int D, int BS, int P, bool kShared>
__global__ __launch_bounds__(64 * kHeadsPerWg) void decode_partition_kernel(DecodeArgs a) {
  using C = DecodeCfg<T, D, BS, P>;
  int hg, s, part;
  if constexpr (kShared) {
    // One-dimensional grid.  Workgroups go to the 8 XCDs round-robin by linear id; here runs
    // of kXcdChunk consecutive work units (sequence fastest, then head group, then partition)
    // stay on one XCD and the runs rotate over the XCDs, so neighbouring sequences - the
    // samples or beams that share blocks - start back to back on one XCD and meet their
    // shared rows in its L2, while every XCD still gets a share of the whole batch.  (With
    // the head group fastest the sharers of a row were a head-group count apart and often
    // in different runs: 7% slower on six samples per prompt.)
    const int hgroups = (a.num_heads + a.heads_per_wg - 1) / a.heads_per_wg;
    const int lin = blockIdx.x;
    const int round = kXcds * kXcdChunk;
    const int full = static_cast<int>(gridDim.x) / round * round;
    int n = lin;
    if (lin < full) {
      const int xcd = lin % kXcds, k = lin / kXcds;
      n = ((k / kXcdChunk) * kXcds + xcd) * kXcdChunk + k % kXcdChunk;
    }
    s = n % a.num_seqs;
    hg = (n / a.num_seqs) % hgroups;
    part = n / (hgroups * a.num_seqs);
  } else {
    // head group fastest, then sequence (longest context first when the launcher ordered
    // them), then partition
    hg = blockIdx.x, part = blockIdx.z;
    s = a.order != nullptr ? a.order[blockIdx.y] : static_cast<int>(blockIdx.y);
  }
  const int h = hg * a.heads_per_wg + static_cast<int>(threadIdx.x >> 6);
  if (h >= a.num_heads) return;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 3;  // token within a group of 8
  const int c = lane & 7;   // 16-byte column within a 128-byte line

  int qrow = s;
  if (a.q_start_loc != nullptr) {
    const int q0 = a.q_start_loc[s];
    if (a.q_start_loc[s + 1] - q0 != 1) return;  // multi-query sequences run the tile path
    qrow = q0;
  }
  if (qrow < 0 || qrow >= a.num_tokens) return;
  const int ctx = min(a.context_lens[s], min(a.max_blocks * BS, a.max_context_len));
  if (ctx <= 0) return;  // malformed length: nothing to read (the merge pass skips it too)
  // with a sliding window the query (position ctx-1) sees tokens lo .. ctx-1; partitions
  // start at the window's first block, so older blocks are never read
  const int lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  const int first = lo / BS * BS;
  const int span = ctx - first;
  const int nparts = (span + P - 1) / P;
  // equal shares (rounded up to whole trips and blocks), so no partition is a short tail
  const int share = ((span + nparts - 1) / nparts + C::kAlign - 1) / C::kAlign * C::kAlign;
  const int start = first + part * share;
  if (start >= ctx) {
    // Rounded-up shares can leave a trailing partition without tokens; the merge pass
    // still reads it, so it records an empty partial (m = -inf, l = 0, acc = 0).
    if (part < nparts && (threadIdx.x & 63) < 8) {
      const int64_t slot = (static_cast<int64_t>(qrow) * a.num_heads + h) * a.num_parts_max + part;
      float* wp = a.ws_acc + slot * D;
      for (int e = (threadIdx.x & 7) * 4; e < D; e += 32)
        st16(wp + e, u32x4{0, 0, 0, 0});
      if ((threadIdx.x & 63) == 0) {
        a.ws_ml[slot * 2] = -INFINITY;
        a.ws_ml[slot * 2 + 1] = 0.f;
      }
    }
    return;
  }
  const int ntok = min(share, ctx - start);

  const int64_t row_stride = static_cast<int64_t>(a.num_heads) * D;
  // element offset of this lane's chunk j inside a head row
  auto col = [&](int j) { return (j * 8 + c) * C::kEpc; };
  const T* kbase = static_cast<const T*>(a.k_pool) + static_cast<int64_t>(h) * D;
  const T* vbase = static_cast<const T*>(a.v_pool) + static_cast<int64_t>(h) * D;

  const T* qp = static_cast<const T*>(a.q) + (static_cast<int64_t>(qrow) * a.num_heads + h) * D;
  u32x4 qc[C::kCpt];
#pragma unroll
  for (int j = 0; j < C::kCpt; ++j) qc[j] = ld16(qp + col(j));

  // physical blocks of this partition, one per lane
  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks + start / BS;
  const int nblk = (ntok + BS - 1) / BS;
  int my_blk[C::kTabRegs];
#pragma unroll
  for (int r = 0; r < C::kTabRegs; ++r) {
    my_blk[r] = 0;
    if (r * kWave + lane < nblk) {
      const int b = btrow[r * kWave + lane];
      my_blk[r] = (b >= 0 && b < a.num_blocks) ? b : 0;
    }
  }
  // row offset of token (group_base + g), where group_base is a multiple of 8 (wave-uniform)
  auto row_offset = [&](int group_base) -> int64_t {
    const int bi = group_base / BS;
    int blk;
    if constexpr (C::kTabRegs == 1) {
      blk = __builtin_amdgcn_readlane(my_blk[0], bi);
    } else {
      blk = bi < kWave ? __builtin_amdgcn_readlane(my_blk[0], bi)
                       : __builtin_amdgcn_readlane(my_blk[C::kTabRegs - 1], bi - kWave);
    }
    return (static_cast<int64_t>(blk) * BS + (group_base % BS) + g) * row_stride;
  };

  float m = -INFINITY, l = 0.f;
  float acc[C::kEpl];
#pragma unroll
  for (int e = 0; e < C::kEpl; ++e) acc[e] = 0.f;

  auto update = [&](const float (&sc)[C::kG], const u32x4 (&vr)[C::kG][C::kCpt],
                    const bool (&ok)[C::kG]) {
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < C::kG; ++i) mx = fmaxf(mx, sc[i]);
    if (__any(mx > m + kTau)) {
      const float mn = fmaxf(m, mx);
      const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < C::kEpl; ++e) acc[e] *= alpha;
      m = mn;
    }
#pragma unroll
    for (int i = 0; i < C::kG; ++i) {
      const float p = ok[i] ? fast_exp2(sc[i] - m) : 0.f;
      l += p;
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j)
#pragma unroll
        for (int e = 0; e < C::kEpc; ++e)
          acc[j * C::kEpc + e] = fmaf(p, chunk_elt<T>(vr[i][j], e), acc[j * C::kEpc + e]);
    }
  };

  // ALiBi: slope * (j - p) added to the score of token j, p = ctx - 1 (log2 units here)
  const float slope = a.alibi != nullptr ? a.alibi[h] * kLog2e : 0.f;
  auto score = [&](const u32x4 (&kr)[C::kCpt], int rel) {
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < C::kCpt; ++j) d = chunk_dot<T>(qc[j], kr[j], d);
    const float x = group_sum<8>(d) * a.scale_log2;
    return fmaf(slope, static_cast<float>(start + rel - (ctx - 1)), x);
  };

  const int full = ntok / C::kTrip;
  for (int trip = 0; trip < full; ++trip) {
    u32x4 kr[C::kG][C::kCpt], vr[C::kG][C::kCpt];
    int64_t off[C::kG];
#pragma unroll
    for (int i = 0; i < C::kG; ++i) {
      off[i] = row_offset(trip * C::kTrip + i * 8);
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j) kr[i][j] = ld_kv<kShared>(kbase + off[i] + col(j));
    }
#pragma unroll
    for (int i = 0; i < C::kG; ++i)
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j) vr[i][j] = ld_kv<kShared>(vbase + off[i] + col(j));
    float sc[C::kG];
    bool ok[C::kG];
    // Only the trips that begin before the window's first token mask anything (the window's
    // first block may start earlier); their masked value rows are cleared so whatever those
    // slots hold gets weight exactly zero.
    const bool head_trip = start + trip * C::kTrip < lo;  // wave-uniform
#pragma unroll
    for (int i = 0; i < C::kG; ++i) {
      const int rel = trip * C::kTrip + i * 8 + g;
      ok[i] = start + rel >= lo;
      const float x = score(kr[i], rel);
      sc[i] = ok[i] ? x : -INFINITY;
    }
    if (head_trip) {
#pragma unroll
      for (int i = 0; i < C::kG; ++i)
#pragma unroll
        for (int j = 0; j < C::kCpt; ++j)
          if (!ok[i]) vr[i][j] = u32x4{0, 0, 0, 0};
    }
    update(sc, vr, ok);
  }

  if (full * C::kTrip < ntok) {  // ragged last trip: lanes past the end load nothing
    u32x4 kr[C::kG][C::kCpt], vr[C::kG][C::kCpt];
    bool ok[C::kG];
#pragma unroll
    for (int i = 0; i < C::kG; ++i) {
      const int base = full * C::kTrip + i * 8;
      ok[i] = base + g < ntok && start + base + g >= lo;
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j) {
        kr[i][j] = u32x4{0, 0, 0, 0};
        vr[i][j] = u32x4{0, 0, 0, 0};
      }
      if (base < ntok) {  // wave-uniform: the group has at least one valid token
        const int64_t off = row_offset(base);
        if (ok[i]) {
#pragma unroll
          for (int j = 0; j < C::kCpt; ++j) kr[i][j] = ld_kv<kShared>(kbase + off + col(j));
#pragma unroll
          for (int j = 0; j < C::kCpt; ++j) vr[i][j] = ld_kv<kShared>(vbase + off + col(j));
        }
      }
    }
    float sc[C::kG];
#pragma unroll
    for (int i = 0; i < C::kG; ++i) {
      const float d = score(kr[i], full * C::kTrip + i * 8 + g);
      sc[i] = ok[i] ? d : -INFINITY;
    }
    update(sc, vr, ok);
  }

  // merge the 8 token groups: common reference, then sum over lanes of equal column c
  const float M = wave_max(m);
  const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
  l *= f;
#pragma unroll
  for (int e = 0; e < C::kEpl; ++e) acc[e] *= f;
#pragma unroll
  for (int x = 8; x < kWave; x <<= 1) {
    l += shfl_xor_f(l, x);
#pragma unroll
    for (int e = 0; e < C::kEpl; ++e) acc[e] += shfl_xor_f(acc[e], x);
  }

  if (g != 0) return;
  if (nparts == 1) {
    const float inv = 1.f / l;
    T* op = static_cast<T*>(a.out) + (static_cast<int64_t>(qrow) * a.num_heads + h) * D;
#pragma unroll
    for (int j = 0; j < C::kCpt; ++j) {
      float v[C::kEpc];
#pragma unroll
      for (int e = 0; e < C::kEpc; ++e) v[e] = acc[j * C::kEpc + e] * inv;
      store_chunk<T>(op + col(j), v);
    }
  } else {
    const int64_t slot = (static_cast<int64_t>(qrow) * a.num_heads + h) * a.num_parts_max + part;
    float* wp = a.ws_acc + slot * D;
#pragma unroll
    for (int j = 0; j < C::kCpt; ++j)
#pragma unroll
      for (int e4 = 0; e4 < C::kEpc; e4 += 4) {
        f32x4 v = {acc[j * C::kEpc + e4], acc[j * C::kEpc + e4 + 1], acc[j * C::kEpc + e4 + 2],
                   acc[j * C::kEpc + e4 + 3]};
        st16(wp + col(j) + e4, __builtin_bit_cast(u32x4, v));
      }
    if (c == 0) {
      a.ws_ml[slot * 2] = M;
      a.ws_ml[slot * 2 + 1] = l;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kPer = D / kWave;  // output elements per lane
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  int qrow = s;
  if (a.q_start_loc != nullptr) {
    const int q0 = a.q_start_loc[s];
    if (a.q_start_loc[s + 1] - q0 != 1) return;
    qrow = q0;
  }
  if (qrow < 0 || qrow >= a.num_tokens) return;
  const int ctx = min(a.context_lens[s], min(a.max_blocks * a.block_size, a.max_context_len));
  const int lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  const int span = ctx - lo / a.block_size * a.block_size;
  const int nparts = min((span + a.part_size - 1) / a.part_size, a.num_parts_max);
  if (nparts <= 1) return;  // pass 1 wrote the output
  const int64_t slot0 = (static_cast<int64_t>(qrow) * a.num_heads + h) * a.num_parts_max;
  const float* ml = a.ws_ml + slot0 * 2;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float L = 0.f;
  float o[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) o[i] = 0.f;
  const float* acc = a.ws_acc + slot0 * D + lane * kPer;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(ml[2 * p] - M);
    L = fmaf(w, ml[2 * p + 1], L);
#pragma unroll
    for (int i = 0; i < kPer; ++i) o[i] = fmaf(w, acc[static_cast<int64_t>(p) * D + i], o[i]);
  }
  const float inv = 1.f / L;
  T* op = static_cast<T*>(a.out) + (static_cast<int64_t>(qrow) * a.num_heads + h) * D + lane * kPer;
#pragma unroll
  for (int i = 0; i < kPer; ++i) op[i] = static_cast<T>(o[i] * inv);
}

// Grouped decode [P1 sec. 6, parallel-sampling and beam-search paragraphs: the samples of
// one prompt share its blocks, beam candidates share their common ancestry].  When the caller
// places such sequences next to each other, in runs of G, their shared rows need only be read
// once for the whole run.  One workgroup of kGroupWaves waves handles one (run, head,
// partition of P tokens); partitions are fixed token ranges [p*P, (p+1)*P), so the members'
// partitions line up.  From the members' context lengths and table entries alone it works out:
//   * the active members: those whose context reaches into the partition;
//   * t = the longest prefix of the partition, in whole trips, that every active member's
//     context covers and whose blocks are the same physical blocks for all of them (at least
//     two active members, else 0);
//   * the work items: the t / kTrip joint trips (each token row read once, through the first
//     active member's entries, and used for every active member), then each active member's
//     own trips from t to the end of its context in the partition (its own entries).
// The items are dealt to the waves round-robin, so the shared rows and the private tails are
// spread over all waves of the workgroup, and each wave's loads run one item ahead of its
// arithmetic (two register buffers).  Every wave keeps a running (m, l, acc) per member; at
// the end the waves' states are merged per member in LDS with the online-softmax rule and the
// member's partial (or, for a single-partition context, its output) is written.  Since the
// split is a function of the tables alone, every (sequence, head, token) is used exactly once,
// through a block equal to its own table entry, whatever the tables hold: a wrong grouping
// costs speed, never correctness.  Partials use the plain kernel's workspace slots and merge.
constexpr int kGroupWaves = 4;

template <int D, int BS, int P, int kCap, bool kAlibi>
__global__ __launch_bounds__(64 * kGroupWaves) void decode_group_kernel(DecodeArgs a) {
  using T = f16;
  using C = DecodeCfg<T, D, BS, P>;
  const int h = blockIdx.x;
  const int lead = static_cast<int>(blockIdx.y) * a.group;
  const int part = blockIdx.z;
  // the wave index, known to the compiler as wave-uniform: the item bookkeeping below then
  // runs on the scalar unit
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 3;  // token within a group of 8
  const int c = lane & 7;   // 16-byte column within a 128-byte line
  const int nmem = min(a.group, a.num_seqs - lead);
  const int cap = min(a.max_blocks * BS, a.max_context_len);
  const int start = part * P;

  // members' clamped context lengths, their tokens in this partition (0: inactive) and their
  // table entries for it; the same values in every thread of the workgroup
  int ctxk[kCap], endk[kCap];
  int blk[kCap][C::kTabRegs];
  int nact = 0, first = -1, reach = P;
#pragma unroll
  for (int k = 0; k < kCap; ++k) {
    ctxk[k] = 0;
    endk[k] = 0;
#pragma unroll
    for (int r = 0; r < C::kTabRegs; ++r) blk[k][r] = 0;
    if (k < nmem) {
      ctxk[k] = min(a.context_lens[lead + k], cap);
      if (ctxk[k] > start) {
        endk[k] = min(ctxk[k] - start, P);
        ++nact;
        if (first < 0) first = k;
        reach = min(reach, endk[k]);
        const int nb = (endk[k] + BS - 1) / BS;
        const int32_t* bt =
            a.block_tables + static_cast<int64_t>(lead + k) * a.max_blocks + start / BS;
#pragma unroll
        for (int r = 0; r < C::kTabRegs; ++r) {
          if (r * kWave + lane < nb) {
            const int b = bt[r * kWave + lane];
            blk[k][r] = (b >= 0 && b < a.num_blocks) ? b : 0;
          }
        }
      }
    }
  }
  if (nact == 0) return;  // the same in every thread: no member has tokens here

  // entries of the first active member: the joint trips read through them
  int fb[C::kTabRegs];
#pragma unroll
  for (int r = 0; r < C::kTabRegs; ++r) {
    fb[r] = 0;
#pragma unroll
    for (int k = 0; k < kCap; ++k)
      if (k == first) fb[r] = blk[k][r];
  }
  int t = 0;  // shared prefix of the partition, in tokens (a multiple of the trip)
  if (nact >= 2) {
    const int nchk = (reach + BS - 1) / BS;  // blocks holding the tokens every member has
    int first_diff = nchk;
#pragma unroll
    for (int r = C::kTabRegs - 1; r >= 0; --r) {
      bool same = true;
#pragma unroll
      for (int k = 0; k < kCap; ++k)
        if (endk[k] > 0) same = same && blk[k][r] == fb[r];
      const uint64_t diff = __ballot(r * kWave + lane < nchk && !same);
      if (diff != 0) first_diff = r * kWave + __builtin_ctzll(diff);
    }
    t = min(first_diff * BS, reach) / C::kTrip * C::kTrip;
  }
  // work items: joint trips [0, nj), then member k's own trips [pstart[k], pstart[k + 1])
  const int nj = t / C::kTrip;
  int pstart[kCap + 1];
  pstart[0] = nj;
#pragma unroll
  for (int k = 0; k < kCap; ++k)
    pstart[k + 1] = pstart[k] + (endk[k] > 0 ? (endk[k] - t + C::kTrip - 1) / C::kTrip : 0);
  const int total = pstart[kCap];

  // the members' query chunks in LDS, one copy per lane slot (written by wave k % kGroupWaves,
  // read by all after the barrier); after them the per-wave states for the final merge
  extern __shared__ u32x4 smem[];
  auto q_slot = [&](int k, int j) -> u32x4& { return smem[(k * C::kCpt + j) * kWave + lane]; };
  auto col = [&](int j) { return (j * 8 + c) * C::kEpc; };
#pragma unroll
  for (int k = 0; k < kCap; ++k) {
    if (endk[k] > 0 && k % kGroupWaves == wv) {
      const T* qp = static_cast<const T*>(a.q) +
                    (static_cast<int64_t>(lead + k) * a.num_heads + h) * D;
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j) q_slot(k, j) = ld16(qp + col(j));
    }
  }
  __syncthreads();

  const int64_t row_stride = static_cast<int64_t>(a.num_heads) * D;
  const T* kbase = static_cast<const T*>(a.k_pool) + static_cast<int64_t>(h) * D;
  const T* vbase = static_cast<const T*>(a.v_pool) + static_cast<int64_t>(h) * D;
  // ALiBi (a compile-time variant): slope * (j - p) added to the score of token j for the
  // member whose query sits at position p (log2 units here)
  const float slope = kAlibi ? a.alibi[h] * kLog2e : 0.f;
  auto score = [&](const u32x4 (&qv)[C::kCpt], const u32x4 (&kr)[C::kCpt], int dist) {
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < C::kCpt; ++j) d = chunk_dot<T>(qv[j], kr[j], d);
    const float x = group_sum<8>(d) * a.scale_log2;
    if constexpr (kAlibi) return fmaf(slope, static_cast<float>(dist), x);
    return x;
  };
  float m[kCap], l[kCap], acc[kCap][C::kEpl];
#pragma unroll
  for (int k = 0; k < kCap; ++k) {
    m[k] = -INFINITY;
    l[k] = 0.f;
#pragma unroll
    for (int e = 0; e < C::kEpl; ++e) acc[k][e] = 0.f;
  }
  auto update = [&](float& mk, float& lk, float (&ak)[C::kEpl], const float (&sc)[C::kG],
                    const u32x4 (&vr)[C::kG][C::kCpt], const bool (&ok)[C::kG]) {
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < C::kG; ++i) mx = fmaxf(mx, sc[i]);
    if (__any(mx > mk + kTau)) {
      const float mn = fmaxf(mk, mx);
      const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(mk - mn);
      lk *= alpha;
#pragma unroll
      for (int e = 0; e < C::kEpl; ++e) ak[e] *= alpha;
      mk = mn;
    }
#pragma unroll
    for (int i = 0; i < C::kG; ++i) {
      const float p = ok[i] ? fast_exp2(sc[i] - mk) : 0.f;
      lk += p;
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j)
#pragma unroll
        for (int e = 0; e < C::kEpc; ++e)
          ak[j * C::kEpc + e] = fmaf(p, chunk_elt<T>(vr[i][j], e), ak[j * C::kEpc + e]);
    }
  };

  // item i (wave-uniform): member k (-1 = joint) and its first token relative to the partition
  auto item = [&](int i, int& k, int& rel) {
    k = -1;
    rel = i * C::kTrip;
#pragma unroll
    for (int kk = 0; kk < kCap; ++kk)
      if (i >= pstart[kk] && i < pstart[kk + 1]) {
        k = kk;
        rel = t + (i - pstart[kk]) * C::kTrip;
      }
  };
  // K and V rows of item i.  Every lane loads a row that holds a token of the member: a lane
  // whose token lies past the member's end (a ragged last trip) reads the member's last token
  // of its 8-token group instead (same block; its weight is zero), and a group wholly past the
  // end reads the group holding the last token.  So the loads need no lane masks.
  auto load = [&](int i, u32x4 (&kr)[C::kG][C::kCpt], u32x4 (&vr)[C::kG][C::kCpt]) {
    int k, rel;
    item(i, k, rel);
    int wb[C::kTabRegs];
    int end = t;
#pragma unroll
    for (int r = 0; r < C::kTabRegs; ++r) wb[r] = fb[r];
#pragma unroll
    for (int kk = 0; kk < kCap; ++kk)
      if (kk == k) {
        end = endk[kk];
#pragma unroll
        for (int r = 0; r < C::kTabRegs; ++r) wb[r] = blk[kk][r];
      }
#pragma unroll
    for (int i8 = 0; i8 < C::kG; ++i8) {
      const int gb = min(rel + i8 * 8, (end - 1) / 8 * 8);  // wave-uniform
      const int bi = gb / BS;
      int id;
      if constexpr (C::kTabRegs == 1) {
        id = __builtin_amdgcn_readlane(wb[0], bi);
      } else {
        id = bi < kWave ? __builtin_amdgcn_readlane(wb[0], bi)
                        : __builtin_amdgcn_readlane(wb[C::kTabRegs - 1], bi - kWave);
      }
      const int tok = min(gb + g, end - 1);
      const int64_t off = (static_cast<int64_t>(id) * BS + tok % BS) * row_stride;
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j) kr[i8][j] = ld_kv<false>(kbase + off + col(j));
    }
#pragma unroll
    for (int i8 = 0; i8 < C::kG; ++i8) {
      const int gb = min(rel + i8 * 8, (end - 1) / 8 * 8);
      const int bi = gb / BS;
      int id;
      if constexpr (C::kTabRegs == 1) {
        id = __builtin_amdgcn_readlane(wb[0], bi);
      } else {
        id = bi < kWave ? __builtin_amdgcn_readlane(wb[0], bi)
                        : __builtin_amdgcn_readlane(wb[C::kTabRegs - 1], bi - kWave);
      }
      const int tok = min(gb + g, end - 1);
      const int64_t off = (static_cast<int64_t>(id) * BS + tok % BS) * row_stride;
#pragma unroll
      for (int j = 0; j < C::kCpt; ++j) vr[i8][j] = ld_kv<false>(vbase + off + col(j));
    }
  };
  // scores and running states of item i from its loaded rows
  auto use = [&](int i, const u32x4 (&kr)[C::kG][C::kCpt], const u32x4 (&vr)[C::kG][C::kCpt]) {
    int k, rel;
    item(i, k, rel);
#pragma unroll
    for (int kk = 0; kk < kCap; ++kk) {
      if (endk[kk] > 0 && (k < 0 || k == kk)) {
        u32x4 qk[C::kCpt];
#pragma unroll
        for (int j = 0; j < C::kCpt; ++j) qk[j] = q_slot(kk, j);
        float sc[C::kG];
        bool ok[C::kG];
#pragma unroll
        for (int i8 = 0; i8 < C::kG; ++i8) {
          const int tok = rel + i8 * 8 + g;
          ok[i8] = tok < endk[kk];
          const float x = score(qk, kr[i8], start + tok - (ctxk[kk] - 1));
          sc[i8] = ok[i8] ? x : -INFINITY;
        }
        update(m[kk], l[kk], acc[kk], sc, vr, ok);
      }
    }
  };

  {
    // three register buffers: the loads of this wave's next two items are in flight while an
    // item is used (with few waves per SIMD, each wave must keep enough bytes in flight)
    // Loads are issued unconditionally (past this wave's last item they re-read it, unused),
    // so every wait for a buffer counts exactly the loads issued after it.
    constexpr int S = kGroupWaves;
    u32x4 ka[C::kG][C::kCpt], va[C::kG][C::kCpt], kb[C::kG][C::kCpt], vb[C::kG][C::kCpt];
    u32x4 kc[C::kG][C::kCpt], vc[C::kG][C::kCpt];
    int i = wv;
    if (i < total) {
      const int last = i + (total - 1 - i) / S * S;  // this wave's last item
      auto nxt = [&](int j) { return j < total ? j : last; };
      load(i, ka, va);
      load(nxt(i + S), kb, vb);
      for (; i < total; i += 3 * S) {
        load(nxt(i + 2 * S), kc, vc);
        use(i, ka, va);
        if (i + S >= total) break;
        load(nxt(i + 3 * S), ka, va);
        use(i + S, kb, vb);
        if (i + 2 * S >= total) break;
        load(nxt(i + 4 * S), kb, vb);
        use(i + 2 * S, kc, vc);
      }
    }
  }

  // each wave's state per member: merge the 8 token groups, then to LDS
  float* mrg_acc = reinterpret_cast<float*>(smem + kCap * C::kCpt * kWave);  // [W][kCap][D]
  float* mrg_ml = mrg_acc + kGroupWaves * kCap * D;                          // [W][kCap][2]
#pragma unroll
  for (int k = 0; k < kCap; ++k) {
    if (endk[k] > 0) {
      const float M = wave_max(m[k]);
      const float f = (m[k] == -INFINITY) ? 0.f : fast_exp2(m[k] - M);
      float lk = l[k] * f;
      float ak[C::kEpl];
#pragma unroll
      for (int e = 0; e < C::kEpl; ++e) ak[e] = acc[k][e] * f;
#pragma unroll
      for (int x = 8; x < kWave; x <<= 1) {
        lk += shfl_xor_f(lk, x);
#pragma unroll
        for (int e = 0; e < C::kEpl; ++e) ak[e] += shfl_xor_f(ak[e], x);
      }
      if (g == 0) {
        float* dst = mrg_acc + (wv * kCap + k) * D;
#pragma unroll
        for (int j = 0; j < C::kCpt; ++j)
#pragma unroll
          for (int e4 = 0; e4 < C::kEpc; e4 += 4) {
            f32x4 v = {ak[j * C::kEpc + e4], ak[j * C::kEpc + e4 + 1], ak[j * C::kEpc + e4 + 2],
                       ak[j * C::kEpc + e4 + 3]};
            *reinterpret_cast<f32x4*>(dst + col(j) + e4) = v;
          }
        if (c == 0) {
          mrg_ml[(wv * kCap + k) * 2] = M;
          mrg_ml[(wv * kCap + k) * 2 + 1] = lk;
        }
      }
    }
  }
  __syncthreads();

  // per member: combine the waves' states, then its output (a context within one partition)
  // or its partial for the merge pass
#pragma unroll
  for (int k = 0; k < kCap; ++k) {
    if (endk[k] == 0) continue;
    float Mw[kGroupWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
      Mw[w] = mrg_ml[(w * kCap + k) * 2];
      M = fmaxf(M, Mw[w]);
    }
    float wt[kGroupWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
      wt[w] = Mw[w] == -INFINITY ? 0.f : fast_exp2(Mw[w] - M);
      L = fmaf(wt[w], mrg_ml[(w * kCap + k) * 2 + 1], L);
    }
    const int64_t row = static_cast<int64_t>(lead + k) * a.num_heads + h;
    const bool single = ctxk[k] <= P;
    for (int d = threadIdx.x; d < D; d += 64 * kGroupWaves) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < kGroupWaves; ++w) o = fmaf(wt[w], mrg_acc[(w * kCap + k) * D + d], o);
      if (single) {
        static_cast<T*>(a.out)[row * D + d] = static_cast<T>(o / L);
      } else {
        const int64_t slot = row * a.num_parts_max + part;
        a.ws_acc[slot * D + d] = o;
        if (d == 0) {
          a.ws_ml[slot * 2] = M;
          a.ws_ml[slot * 2 + 1] = L;
        }
      }
    }
  }
}

size_t decode_workspace_bytes(int64_t num_tokens, int64_t num_heads, int64_t head_dim,
                              int64_t max_context_len) {
  const int64_t nparts = workspace_parts(static_cast<int>(max_context_len));
  if (nparts <= 1) return 0;
  // partials (accumulators, then (max, sum) pairs), then one int per query row for the
  // longest-first order of the sequences
  return static_cast<size_t>(num_tokens * num_heads * nparts * (head_dim + 2) * 4 +
                             num_tokens * 4);
}

// Longest-first order of the sequences for pass 1 [a scheduling choice, not part of the
// method: the partitions of the longest contexts start first, so the launch does not end on
// them].  Sequence j's key is (clamped length << 32) | ~j: keys are distinct, and a larger key
// means a longer context, or an equal one and a smaller index.  Sequence t's rank = the number
// of keys above its own (so the ranks are a permutation), and order[rank] = t.  Workgroup b
// ranks sequences 64b..64b+63, one per lane; each of its four waves counts over a quarter of
// the keys (staged in LDS), and the quarters' counts are summed in LDS.
constexpr int kOrderMaxSeqs = 1024;
constexpr int kOrderWaves = 4;

__global__ __launch_bounds__(kWave * kOrderWaves) void decode_order_kernel(
    const int32_t* context_lens, int num_seqs, int cap, int32_t* order) {
  __shared__ uint64_t key[kOrderMaxSeqs];
  __shared__ int part[kOrderWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // slots past num_seqs (up to the quarter boundary) hold 0, below every real key
  const int quarter = ((num_seqs + kOrderWaves - 1) / kOrderWaves + 7) & ~7;
  for (int j = threadIdx.x; j < quarter * kOrderWaves; j += kWave * kOrderWaves) {
    uint64_t k = 0;
    if (j < num_seqs) {
      const uint32_t len = static_cast<uint32_t>(min(max(context_lens[j], 0), cap));
      k = (static_cast<uint64_t>(len) << 32) | static_cast<uint32_t>(~j);
    }
    key[j] = k;
  }
  __syncthreads();
  const int t = blockIdx.x * kWave + lane;
  const uint64_t mine = t < num_seqs ? key[t] : ~0ull;
  int count = 0;
  for (int j0 = wv * quarter; j0 < (wv + 1) * quarter; j0 += 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) count += key[j0 + e] > mine ? 1 : 0;
  }
  part[wv][lane] = count;
  __syncthreads();
  if (wv == 0 && t < num_seqs) {
    int rank = 0;
#pragma unroll
    for (int w = 0; w < kOrderWaves; ++w) rank += part[w][lane];
    order[rank] = t;
  }
}

// Order the sequences longest first when the launch is long enough for its tail to matter
// (measured on MI355X: 256 sequences x 40 heads with contexts U{1025..4097}, 13.4 GB: 1.99 vs
// 2.07 ms; 64 sequences x 40 heads, lognormal lengths, 1 GB: within 1%, less than the extra
// launch costs): at least kOrderMinBytes of K/V as bounded by the longest context, more than
// one partition, and no sliding window (a window caps every sequence's span, so the lengths
// stop mattering: the same large batch with a 1,024-token window, 0.845 ms ordered vs 0.836).
constexpr double kOrderMinBytes = 4e9;

// Longest token span one (sequence, head) reads: the context, or with a sliding window
// the window plus the part of its first block that precedes it.
static int decode_span(const DecodeArgs& a, int block_size, int max_context_len) {
  if (a.window <= 0) return max_context_len;
  return max_context_len < a.window + block_size - 1 ? max_context_len : a.window + block_size - 1;
}

template <typename T, int D, int BS, int P>
static hipError_t launch_decode_t(const DecodeArgs& a0, int max_context_len, hipStream_t stream) {
  DecodeArgs a = a0;
  a.part_size = P;
  const int nparts = (decode_span(a, BS, max_context_len) + P - 1) / P;
  // slots at the workspace's common stride (P >= kMinPartition, so nparts fits); ws_ml
  // follows ws_acc
  a.num_parts_max = workspace_parts(max_context_len);
  a.ws_acc = static_cast<float*>(a.workspace);
  a.ws_ml = a.ws_acc + static_cast<int64_t>(a.num_tokens) * a.num_heads * a.num_parts_max * D;
  a.heads_per_wg = a.num_heads % kHeadsPerWg == 0 ? kHeadsPerWg : 1;
  const int hgroups = a.num_heads / a.heads_per_wg;
  const dim3 block1(kWave * a.heads_per_wg);
  a.order = nullptr;
  if (a.flags & kDecodeSharedBlocks) {
    dim3 grid1(static_cast<unsigned>(hgroups) * a.num_seqs * nparts);
    hipLaunchKernelGGL((decode_partition_kernel<T, D, BS, P, true>), grid1, block1, 0, stream,
                       a);
  } else {
    const double bound =
        static_cast<double>(a.num_seqs) * a.num_heads * max_context_len * 2.0 * D * sizeof(T);
    // the order takes num_seqs of the num_tokens ints after the partials
    if (a.workspace != nullptr && a.window <= 0 && nparts > 1 && a.num_seqs > 1 &&
        a.num_seqs <= kOrderMaxSeqs && a.num_seqs <= a.num_tokens && bound >= kOrderMinBytes) {
      int32_t* order = reinterpret_cast<int32_t*>(
          a.ws_ml + static_cast<int64_t>(a.num_tokens) * a.num_heads * a.num_parts_max * 2);
      const int cap = static_cast<int>(
          std::min<int64_t>(static_cast<int64_t>(a.max_blocks) * BS, max_context_len));
      const unsigned wgs = static_cast<unsigned>((a.num_seqs + kWave - 1) / kWave);
      hipLaunchKernelGGL(decode_order_kernel, dim3(wgs), dim3(kWave * kOrderWaves), 0, stream,
                         a.context_lens, a.num_seqs, cap, order);
      a.order = order;
    }
    dim3 grid1(hgroups, a.num_seqs, nparts);
    hipLaunchKernelGGL((decode_partition_kernel<T, D, BS, P, false>), grid1, block1, 0, stream,
                       a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nparts <= 1) return err;
  dim3 grid2(a.num_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), grid2, dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

// Largest partition (fewest partial results) that still gives the launch enough waves
// to fill the chip: sequences x heads x partitions of the longest context >= kTargetWaves.
// The table preload holds at most 128 block ids, which caps the partition for B = 8.
constexpr int64_t kTargetWaves = 16384;

static int pick_partition(const DecodeArgs& a, int block_size, int max_context_len) {
  const int cap = block_size == 8 ? 1024 : 2048;
  const int64_t units = static_cast<int64_t>(a.num_seqs) * a.num_heads;
  int p = cap;
  while (p > kMinPartition && units * ((max_context_len + p - 1) / p) < kTargetWaves) p >>= 1;
  return p;
}

template <typename T, int D, int BS>
static hipError_t launch_decode_p(const DecodeArgs& a, int max_context_len, hipStream_t stream) {
  const int p = pick_partition(a, BS, decode_span(a, BS, max_context_len));
  constexpr int kCapP = BS == 8 ? 1024 : 2048;
  switch (p < kCapP ? p : kCapP) {
    case 256: return launch_decode_t<T, D, BS, 256>(a, max_context_len, stream);
    case 512: return launch_decode_t<T, D, BS, 512>(a, max_context_len, stream);
    case 1024: return launch_decode_t<T, D, BS, 1024>(a, max_context_len, stream);
    default: return launch_decode_t<T, D, BS, kCapP>(a, max_context_len, stream);
  }
}

template <typename T, int D>
static hipError_t launch_decode_bs(const DecodeArgs& a, int block_size, int max_context_len,
                                   hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_decode_p<T, D, 8>(a, max_context_len, stream);
    case 16: return launch_decode_p<T, D, 16>(a, max_context_len, stream);
    case 32: return launch_decode_p<T, D, 32>(a, max_context_len, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int BS, int P, int kCap, bool kAlibi>
static hipError_t launch_group_t(const DecodeArgs& a0, int max_context_len, hipStream_t stream) {
  DecodeArgs a = a0;
  a.part_size = P;
  const int nparts = (max_context_len + P - 1) / P;
  a.num_parts_max = workspace_parts(max_context_len);
  a.ws_acc = static_cast<float*>(a.workspace);
  a.ws_ml = a.ws_acc + static_cast<int64_t>(a.num_tokens) * a.num_heads * a.num_parts_max * D;
  const int runs = (a.num_seqs + a.group - 1) / a.group;
  const dim3 grid1(a.num_heads, runs, nparts);
  // LDS: the members' query chunks (one per lane slot) and the waves' states for the merge
  const size_t lds = static_cast<size_t>(kCap) * (D * 2 / 128) * kWave * 16 +
                     static_cast<size_t>(kGroupWaves) * kCap * (D + 2) * 4;
  hipLaunchKernelGGL((decode_group_kernel<D, BS, P, kCap, kAlibi>), grid1,
                     dim3(kWave * kGroupWaves), lds, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nparts <= 1) return err;
  hipLaunchKernelGGL((decode_merge_kernel<f16, D>), dim3(a.num_heads, a.num_seqs), dim3(kWave), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int BS, int P, bool kAlibi>
static hipError_t launch_group_cap(const DecodeArgs& a, int max_context_len, hipStream_t stream) {
  if (a.group <= 2) return launch_group_t<D, BS, P, 2, kAlibi>(a, max_context_len, stream);
  if (a.group <= 4) return launch_group_t<D, BS, P, 4, kAlibi>(a, max_context_len, stream);
  return launch_group_t<D, BS, P, kMaxDecodeGroup, kAlibi>(a, max_context_len, stream);
}

template <int D, int BS, int P>
static hipError_t launch_group_cap(const DecodeArgs& a, int max_context_len, hipStream_t stream) {
  if (a.alibi != nullptr) return launch_group_cap<D, BS, P, true>(a, max_context_len, stream);
  return launch_group_cap<D, BS, P, false>(a, max_context_len, stream);
}

// Grouped decode partition: the largest of 2048 (block size >= 16), 1024 and 512 tokens for
// which runs x heads x partitions of the longest context reach kGroupTargetWgs workgroups
// (about two rounds of the chip at two workgroups per CU), else 512.  Longer partitions give
// each wave more items for the same per-workgroup set-up and merge.  Measured on MI355X:
// 16 runs of 6 samples x 40 heads (contexts up to ~1,300) fastest at 1024; the same batch at
// 5 heads at 512; 64 runs of 4 or 6 beams x 40 heads (contexts up to ~4,200) at 2048.
constexpr int64_t kGroupTargetWgs = 1024;

static int pick_group_partition(const DecodeArgs& a, int block_size, int max_context_len) {
  const int64_t units =
      static_cast<int64_t>((a.num_seqs + a.group - 1) / a.group) * a.num_heads;
  int p = block_size == 8 ? 1024 : 2048;
  while (p > 512 && units * ((max_context_len + p - 1) / p) < kGroupTargetWgs) p >>= 1;
  return p;
}

template <int D, int BS>
static hipError_t launch_group_p(const DecodeArgs& a, int max_context_len, hipStream_t stream) {
  const int p = pick_group_partition(a, BS, max_context_len);
  if (p <= 512) return launch_group_cap<D, BS, 512>(a, max_context_len, stream);
  if constexpr (BS == 8) {
    return launch_group_cap<D, BS, 1024>(a, max_context_len, stream);
  } else {
    if (p <= 1024) return launch_group_cap<D, BS, 1024>(a, max_context_len, stream);
    return launch_group_cap<D, BS, 2048>(a, max_context_len, stream);
  }
}

// Grouped decode (fp16, no window, one query per sequence; checked by the caller).
template <int D>
static hipError_t launch_group(const DecodeArgs& a, int block_size, int max_context_len,
                               hipStream_t stream) {
  static_assert(kMaxDecodeGroup == 6, "group capacities below are 2, 4 and 6");
  switch (block_size) {
    case 8: return launch_group_p<D, 8>(a, max_context_len, stream);
    case 16: return launch_group_p<D, 16>(a, max_context_len, stream);
    case 32: return launch_group_p<D, 32>(a, max_context_len, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                         int max_context_len, hipStream_t stream) {
  if (a.group > 1) {
    if (dtype != 1 || a.window != 0 || a.q_start_loc != nullptr || a.group > kMaxDecodeGroup)
      return hipErrorInvalidValue;
    if (head_dim == 128) return launch_group<128>(a, block_size, max_context_len, stream);
    if (head_dim == 64) return launch_group<64>(a, block_size, max_context_len, stream);
    return hipErrorInvalidValue;
  }
  if (dtype == 1) {
    if (head_dim == 128) return launch_decode_bs<f16, 128>(a, block_size, max_context_len, stream);
    if (head_dim == 64) return launch_decode_bs<f16, 64>(a, block_size, max_context_len, stream);
  } else {
    if (head_dim == 128) return launch_decode_bs<float, 128>(a, block_size, max_context_len, stream);
    if (head_dim == 64) return launch_decode_bs<float, 64>(a, block_size, max_context_len, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
