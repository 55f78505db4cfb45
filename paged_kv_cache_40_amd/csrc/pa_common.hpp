// Device helpers shared by the gfx950 kernels of the paged KV-cache library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Streaming 16-byte load: the data is read once, so hint the caches not to keep it.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// DPP lane moves inside a row of 16 lanes (quad_perm / mirror controls).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i inside each half row
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i inside each row

// Sum over aligned groups of N consecutive lanes (N in 1,2,4,8,16); every lane of a
// group receives the group total.  After the xor-1/xor-2 steps all lanes of a quad
// hold the same value, so the mirror steps pair whole quads / half rows.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_mov<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_mov<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element e (0-based) of a 16-byte chunk, as fp32.
template <typename T>
__device__ __forceinline__ float chunk_elt(const u32x4& c, int e);

template <>
__device__ __forceinline__ float chunk_elt<f16>(const u32x4& c, int e) {
  f16x8 h = __builtin_bit_cast(f16x8, c);
  return static_cast<float>(h[e]);
}

template <>
__device__ __forceinline__ float chunk_elt<float>(const u32x4& c, int e) {
  f32x4 f = __builtin_bit_cast(f32x4, c);
  return f[e];
}

// Partial dot product of one 16-byte chunk of q with one of k, accumulated in fp32.
template <typename T>
__device__ __forceinline__ float chunk_dot(const u32x4& q, const u32x4& k, float acc);

// Note: the dwords are copied into plain arrays first.  __builtin_bit_cast applied
// directly to a subscripted vector element (q[i]) reads element 0 for every i
// with this compiler, which silently turns the dot product into 4x one term.
template <>
__device__ __forceinline__ float chunk_dot<f16>(const u32x4& q, const u32x4& k, float acc) {
  const uint32_t qa[4] = {q.x, q.y, q.z, q.w};
  const uint32_t ka[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qa[i]), __builtin_bit_cast(f16x2, ka[i]),
                                 acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<float>(const u32x4& q, const u32x4& k, float acc) {
  const f32x4 qf = __builtin_bit_cast(f32x4, q);
  const f32x4 kf = __builtin_bit_cast(f32x4, k);
  const float qa[4] = {qf.x, qf.y, qf.z, qf.w};
  const float ka[4] = {kf.x, kf.y, kf.z, kf.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(qa[i], ka[i], acc);
  return acc;
}

// Store n consecutive fp32 values as T (n = elements of one 16-byte chunk of T).
template <typename T>
__device__ __forceinline__ void store_chunk(T* dst, const float* v);

template <>
__device__ __forceinline__ void store_chunk<f16>(f16* dst, const float* v) {
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = static_cast<f16>(v[i]);
  st16(dst, __builtin_bit_cast(u32x4, h));
}

template <>
__device__ __forceinline__ void store_chunk<float>(float* dst, const float* v) {
  f32x4 f = {v[0], v[1], v[2], v[3]};
  st16(dst, __builtin_bit_cast(u32x4, f));
}

}  // namespace pa
