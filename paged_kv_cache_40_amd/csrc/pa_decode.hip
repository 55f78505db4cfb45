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
// Pass 1: one 64-lane workgroup per (sequence, head, partition of P tokens).
//   * A token's head row (d elements) is split over kLpt lanes, 64 bytes
//     each, fetched as four 16-byte loads arranged so that the kLpt lanes of
//     a token read contiguous 16*kLpt-byte segments per instruction; one
//     iteration covers kTpi = 64/kLpt tokens, a trip covers kU iterations and
//     issues all of its K and V loads before using any of them.
//   * q.k: v_dot2_f32_f16 (fp16) or fma (fp32) over the lane's 64 bytes, then a
//     DPP sum over the token's kLpt lanes (quad_perm / row mirrors).
//   * Softmax runs in the log2 domain (scores pre-multiplied by log2(e)/sqrt(d),
//     v_exp_f32).  Each lane keeps (m, l, acc) for its own token positions;
//     the running reference m only moves when some lane sees a score more
//     than kTau above it (a wave vote), since any reference gives the same
//     ratio and exponents stay below 2^kTau.
//   * At the end the lanes are merged to one (m, l, acc[d]); a sequence with a
//     single partition writes the normalised output directly.
// Pass 2: one 64-lane workgroup per (sequence, head) with more than one
//   partition merges the partials and writes out.
//
// Block ids of a partition are loaded once (one per lane) and broadcast with
// readlane / bpermute.  All pool offsets are 64-bit.  Context lengths are
// clamped to the table width and block ids outside [0, num_blocks) are
// replaced by block 0, so malformed device data cannot address memory
// outside the pools.

#include <math.h>

#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

template <typename T, int D, int BS, int P>
struct DecodeCfg {
  static constexpr int kElt = sizeof(T);
  static constexpr int kRow = D * kElt;        // bytes of one head's row of one token
  static constexpr int kLpt = kRow / 64;       // lanes per token (64 bytes each)
  static constexpr int kTpi = kWave / kLpt;    // tokens per iteration
  static constexpr int kEpc = 16 / kElt;       // elements per 16-byte chunk
  static constexpr int kEpl = 4 * kEpc;        // elements per lane per token
  static constexpr int kU = kTpi >= 32 ? 1 : 2;  // iterations per trip
  static constexpr int kTrip = kU * kTpi;      // tokens per trip
  static constexpr int kBlocks = P / BS;       // table entries per partition
  static constexpr bool kUniformBlock = (BS % kTpi) == 0;  // one block per iteration
  static_assert(kLpt >= 2 && kLpt <= 8, "row must span 2..8 lanes");
  static_assert(P % kTrip == 0 && P % BS == 0, "partition must hold whole trips and blocks");
  static_assert(kBlocks <= kWave, "one table entry per lane");
};

constexpr float kTau = 8.0f;  // log2 headroom before the running reference moves

template <typename T, int D, int BS, int P>
__global__ __launch_bounds__(64) void decode_partition_kernel(DecodeArgs a) {
  using C = DecodeCfg<T, D, BS, P>;
  const int h = blockIdx.x;
  const int part = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int tok = lane / C::kLpt;
  const int c = lane % C::kLpt;

  int qrow = s;
  if (a.q_start_loc != nullptr) {
    const int q0 = a.q_start_loc[s];
    if (a.q_start_loc[s + 1] - q0 != 1) return;  // multi-query sequences run the tile path
    qrow = q0;
  }
  if (qrow < 0 || qrow >= a.num_tokens) return;
  const int ctx = min(a.context_lens[s], min(a.max_blocks * BS, a.max_context_len));
  const int start = part * P;
  if (start >= ctx) return;
  const int ntok = min(P, ctx - start);
  const int nparts = (ctx + P - 1) / P;

  const int64_t row_stride = static_cast<int64_t>(a.num_heads) * D;
  const T* kbase = static_cast<const T*>(a.k_pool) + static_cast<int64_t>(h) * D;
  const T* vbase = static_cast<const T*>(a.v_pool) + static_cast<int64_t>(h) * D;

  // this lane's four chunks of q
  const T* qp = static_cast<const T*>(a.q) + (static_cast<int64_t>(qrow) * a.num_heads + h) * D;
  u32x4 qc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) qc[k] = ld16(qp + (k * C::kLpt + c) * C::kEpc);

  // physical blocks of this partition, one per lane
  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks + start / BS;
  const int nblk = (ntok + BS - 1) / BS;
  int my_blk = 0;
  if (lane < nblk) {
    const int b = btrow[lane];
    my_blk = (b >= 0 && b < a.num_blocks) ? b : 0;
  }

  auto token_offset = [&](int jrel) -> int64_t {
    int blk;
    if constexpr (C::kUniformBlock) {
      blk = __builtin_amdgcn_readlane(my_blk, __builtin_amdgcn_readfirstlane(jrel / BS));
    } else {
      blk = __shfl(my_blk, jrel / BS, kWave);
    }
    return (static_cast<int64_t>(blk) * BS + (jrel % BS)) * row_stride;
  };

  float m = -INFINITY, l = 0.f;
  float acc[C::kEpl];
#pragma unroll
  for (int e = 0; e < C::kEpl; ++e) acc[e] = 0.f;

  auto update = [&](const float (&sc)[C::kU], const u32x4 (&vr)[C::kU][4], const bool (&ok)[C::kU]) {
    float mx = sc[0];
#pragma unroll
    for (int u = 1; u < C::kU; ++u) mx = fmaxf(mx, sc[u]);
    if (__any(mx > m + kTau)) {
      const float mn = fmaxf(m, mx);
      const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < C::kEpl; ++e) acc[e] *= alpha;
      m = mn;
    }
#pragma unroll
    for (int u = 0; u < C::kU; ++u) {
      const float p = ok[u] ? fast_exp2(sc[u] - m) : 0.f;
      l += p;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < C::kEpc; ++e)
          acc[k * C::kEpc + e] = fmaf(p, chunk_elt<T>(vr[u][k], e), acc[k * C::kEpc + e]);
    }
  };

  const int full = ntok / C::kTrip;
  for (int trip = 0; trip < full; ++trip) {
    u32x4 kr[C::kU][4], vr[C::kU][4];
    int64_t off[C::kU];
#pragma unroll
    for (int u = 0; u < C::kU; ++u) {
      off[u] = token_offset((trip * C::kU + u) * C::kTpi + tok);
#pragma unroll
      for (int k = 0; k < 4; ++k) kr[u][k] = ld16(kbase + off[u] + (k * C::kLpt + c) * C::kEpc);
    }
#pragma unroll
    for (int u = 0; u < C::kU; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) vr[u][k] = ld16(vbase + off[u] + (k * C::kLpt + c) * C::kEpc);
    float sc[C::kU];
    bool ok[C::kU];
#pragma unroll
    for (int u = 0; u < C::kU; ++u) {
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) d = chunk_dot<T>(qc[k], kr[u][k], d);
      sc[u] = group_sum<C::kLpt>(d) * a.scale_log2;
      ok[u] = true;
    }
    update(sc, vr, ok);
  }

  if (full * C::kTrip < ntok) {  // ragged last trip: lanes past the end load nothing
    u32x4 kr[C::kU][4], vr[C::kU][4];
    bool ok[C::kU];
    int64_t off[C::kU];
#pragma unroll
    for (int u = 0; u < C::kU; ++u) {
      const int jrel = (full * C::kU + u) * C::kTpi + tok;
      ok[u] = jrel < ntok;
      off[u] = token_offset(ok[u] ? jrel : 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        kr[u][k] = u32x4{0, 0, 0, 0};
        vr[u][k] = u32x4{0, 0, 0, 0};
      }
      if (ok[u]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) kr[u][k] = ld16(kbase + off[u] + (k * C::kLpt + c) * C::kEpc);
#pragma unroll
        for (int k = 0; k < 4; ++k) vr[u][k] = ld16(vbase + off[u] + (k * C::kLpt + c) * C::kEpc);
      }
    }
    float sc[C::kU];
#pragma unroll
    for (int u = 0; u < C::kU; ++u) {
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) d = chunk_dot<T>(qc[k], kr[u][k], d);
      d = group_sum<C::kLpt>(d) * a.scale_log2;
      sc[u] = ok[u] ? d : -INFINITY;
    }
    update(sc, vr, ok);
  }

  // merge the lanes: common reference, then sum over the token lanes of each chunk index
  const float M = wave_max(m);
  const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
  l *= f;
#pragma unroll
  for (int e = 0; e < C::kEpl; ++e) acc[e] *= f;
#pragma unroll
  for (int x = C::kLpt; x < kWave; x <<= 1) {
    l += shfl_xor_f(l, x);
#pragma unroll
    for (int e = 0; e < C::kEpl; ++e) acc[e] += shfl_xor_f(acc[e], x);
  }

  if (tok != 0) return;
  if (nparts == 1) {
    const float inv = 1.f / l;
    T* op = static_cast<T*>(a.out) + (static_cast<int64_t>(qrow) * a.num_heads + h) * D;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v[C::kEpc];
#pragma unroll
      for (int e = 0; e < C::kEpc; ++e) v[e] = acc[k * C::kEpc + e] * inv;
      store_chunk<T>(op + (k * C::kLpt + c) * C::kEpc, v);
    }
  } else {
    const int64_t slot = (static_cast<int64_t>(qrow) * a.num_heads + h) * a.num_parts_max + part;
    float* wp = a.ws_acc + slot * D;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e4 = 0; e4 < C::kEpc; e4 += 4) {
        f32x4 v = {acc[k * C::kEpc + e4], acc[k * C::kEpc + e4 + 1], acc[k * C::kEpc + e4 + 2],
                   acc[k * C::kEpc + e4 + 3]};
        st16(wp + (k * C::kLpt + c) * C::kEpc + e4, __builtin_bit_cast(u32x4, v));
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
  const int nparts = min((ctx + a.part_size - 1) / a.part_size, a.num_parts_max);
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

size_t decode_workspace_bytes(int64_t num_tokens, int64_t num_heads, int64_t head_dim,
                              int64_t max_context_len) {
  const int64_t nparts = (max_context_len + kMinPartition - 1) / kMinPartition;
  if (nparts <= 1) return 0;
  return static_cast<size_t>(num_tokens * num_heads * nparts * (head_dim + 2) * 4);
}

template <typename T, int D, int BS, int P>
static hipError_t launch_decode_t(const DecodeArgs& a0, int max_context_len, hipStream_t stream) {
  DecodeArgs a = a0;
  a.part_size = P;
  const int nparts = (max_context_len + P - 1) / P;
  a.num_parts_max = nparts;
  a.ws_acc = static_cast<float*>(a.workspace);
  a.ws_ml = a.ws_acc + static_cast<int64_t>(a.num_tokens) * a.num_heads * nparts * D;
  dim3 grid1(a.num_heads, nparts, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, BS, P>), grid1, dim3(kWave), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nparts <= 1) return err;
  dim3 grid2(a.num_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), grid2, dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_bs(const DecodeArgs& a, int block_size, int max_context_len,
                                   hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_decode_t<T, D, 8, kMinPartition>(a, max_context_len, stream);
    case 16: return launch_decode_t<T, D, 16, kMinPartition>(a, max_context_len, stream);
    case 32: return launch_decode_t<T, D, 32, kMinPartition>(a, max_context_len, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                         int max_context_len, hipStream_t stream) {
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
